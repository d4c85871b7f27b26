"""The benchmark's algorithmic byte and FLOP counts (the numerators of its
roofline figures) checked against counts taken another way: cache tiles and
stored rows enumerated from the page layout, unmasked (query, key) pairs
counted one by one, and the counter summary's copy calibration on a
synthetic profile directory."""
import csv
import math
import os

import numpy as np
import pytest

import bench
import datagen

W = datagen.WORKLOADS


@pytest.mark.parametrize("name", ["cla2_64k", "tinyllama_cla2", "depthgraft", "tiny_cla2"])
def test_dense_decode_bytes_are_every_source_tile_once(name):
    wl = W[name]
    src, _ = datagen.share_map(wl)
    elem = 4 if wl.dtype == "f32" else 2
    assert wl.ctx % 64 == 0
    pages = wl.ctx // 64
    for l in range(wl.n_layers):
        n_src = 1 if int(src[l, 1]) < 0 else 2
        # K and V tiles of 64 keys x hd, per (sequence, KV head, page, source)
        tiles = wl.batch * wl.n_kv_heads * pages * n_src * 2
        assert bench.bytes_per_call(wl, src, l) == tiles * 64 * wl.head_dim * elem
    if name == "cla2_64k":
        # the default line's launch: 4 x 8 heads x 64K keys x 128 dims x K,V x bf16 = 1 GiB
        assert bench.bytes_per_call(wl, src, 0) == 1 << 30


def test_factorized_decode_bytes_are_the_stored_rows():
    wl = W["factorized_64k"]
    rank = datagen.token_ranks(wl)
    r = rank.numpy().astype(np.int64)
    assert set(np.unique(r)) <= {0, 8, 16}
    pages = wl.ctx // 64
    Hkv, R = wl.n_kv_heads, wl.basis_rank
    # per (sequence, page, KV head): the cK and cV pages (64 x R bf16 each) and
    # both fp16 scale rows (64 each); the codes a token owns in the K and the
    # V blob: ceil(r/8) granules of 8 bytes; one rank byte per (sequence, token)
    coef = wl.batch * pages * Hkv * 2 * 64 * R * 2
    scales = wl.batch * pages * Hkv * 2 * 64 * 2
    granules = sum(math.ceil(int(x) / 8) for x in r.reshape(-1))
    codes = Hkv * 2 * 8 * granules
    ranks = wl.batch * wl.ctx
    assert bench.fact_bytes_per_call(wl, rank) == coef + scales + codes + ranks
    assert bench.algorithmic_bytes(wl, "fact_decode_kernel<128, 4, false>") == coef + scales + codes + ranks


def _unmasked_pairs(n, T):
    # query i of the chunk sits at T - n + i and sees keys 0 .. T - n + i
    return sum(T - n + i + 1 for i in range(n))


@pytest.mark.parametrize("n,T", [(1, 1), (5, 9), (64, 64), (37, 200)])
def test_prefill_flops_count_unmasked_pairs(n, T):
    pairs = sum(1 for i in range(n) for j in range(T) if j <= T - n + i)
    assert pairs == _unmasked_pairs(n, T)
    assert bench.prefill_flops(n, T, 3, 64) == pairs * 3 * (2 * 64 + 2 * 64)
    # coefficient space: 2 x 48 per pair for the score and for the values,
    # 2 x hd x 48 per query row at each end
    assert bench.fact_prefill_flops(n, T, 3, 64) == 3 * (pairs * 4 * 48 + n * 4 * 64 * 48)


def test_prefill_chunk_flops_of_the_benchmark():
    wl = bench.prefill_wl("depthgraft_prefill_chunk")
    pairs = _unmasked_pairs(wl.prefill_n, wl.ctx)
    assert pairs == 4096 * 4096 + 4096 * 4097 // 2
    assert bench.prefill_kernel_flops(wl, "prefill_kernel") == pairs * wl.n_q_heads * 4 * wl.head_dim


def test_issue_roofline_peak():
    # dense: 6.5 VALU slots per pair at half the fp32 FLOP rate (one lane-op
    # per slot), plus 4 * hd MFMA FLOPs at the bf16 peak, serialised
    wl = bench.prefill_wl("depthgraft_prefill_chunk")
    got = bench.issue_roofline(wl, False, 1000.0)
    per_pair_s = 6.5 / (157.3e12 / 2) + 4 * wl.head_dim / 2.5e15
    assert got["peak"] == pytest.approx(1.0 / per_pair_s, rel=1e-12)
    pairs = wl.n_q_heads * _unmasked_pairs(wl.prefill_n, wl.ctx)
    assert got["achieved"] == pytest.approx(pairs / 1e-3, rel=1e-12)


def test_issue_roofline_peak_factorized():
    # factorized: per 64-key page a wave of 32 query rows issues 6 score
    # products (2 key blocks x 3 steps over the 48 coefficients) and 8 value
    # products (2 column blocks x 4 key steps), each a 32 x 32 x 16 MFMA
    wl = bench.prefill_wl("factorized_prefill_chunk")
    flops_per_pair = (6 + 8) * 2 * 32 * 32 * 16 / (32 * 64)
    got = bench.issue_roofline(wl, True, 1000.0)
    assert got["mfma_flops_per_pair_issued"] == flops_per_pair
    per_pair_s = 6.5 / (157.3e12 / 2) + flops_per_pair / 2.5e15
    assert got["peak"] == pytest.approx(1.0 / per_pair_s, rel=1e-12)


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_summary_copy_calibration(tmp_path):
    # a profile directory as rocprofv3 writes it: the named kernel twice, one
    # other kernel, and the 256 MiB reference copy whose FETCH_SIZE reads half
    # its bytes (the gfx950 behaviour the calibration corrects)
    k = "kvs::(anonymous namespace)::decode_kernel<unsigned short, 128, 4, 1>(kvs::(anonymous namespace)::DecodeParams)"
    _write_csv(str(tmp_path / "kt" / "run_kernel_stats.csv"), ["Name", "Calls", "TotalDurationNs"],
               [[k, 2, 300000], ["other_kernel", 5, 10]])
    copy_kib = (256 << 20) / 1024 / 2
    for sub, counter, mine in (("fetch", "FETCH_SIZE", 500000.0), ("write", "WRITE_SIZE", 100.0)):
        _write_csv(str(tmp_path / sub / "run_counter_collection.csv"),
                   ["Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[k, counter, mine], [k, counter, mine], ["other_kernel", counter, 7.0],
                    ["__amd_rocclr_copyBuffer", counter, copy_kib]])
    s = bench.summarize(str(tmp_path), "decode_kernel<unsigned short, 128, 4, 1>", "cla2_64k")
    assert s["calls"] == 2 and s["avg_us"] == pytest.approx(150.0)
    assert s["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert s["FETCH_SIZE"]["bytes_per_dispatch"] == pytest.approx(500000.0 * 1024 * 2.0)
    assert s["WRITE_SIZE"]["bytes_per_dispatch"] == pytest.approx(100.0 * 1024 * 2.0)


@pytest.mark.parametrize("extra", [[], ["--workload", "depthgraft_prefill_chunk"], ["--sweep"],
                                   ["--workload", "factorized_encode_chunk"]])
def test_bench_refuses_more_than_one_gpu(extra):
    # every mode exits with status 2 and says why, before touching a GPU
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"] + extra,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
