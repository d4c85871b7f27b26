"""GPU parity of the dense shared-KV path (append + split-K decode + combine)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from tests._gpu_harness import Dense, assert_close, errors, note, TOL_ABS

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS

CASES = {
    # name: (workload, batch, ctx, lens)
    "tiny_cla2_full": (W["tiny_cla2"], 1, 128, [128]),
    "tiny_cla2_ragged": (W["tiny_cla2"], 3, 128, [128, 1, 65]),
    "tinyllama_shape_ragged": (W["tinyllama_cla2"].with_(n_layers=4), 3, 300, [300, 131, 64]),
    "depthgraft_small_map": (W["depthgraft"].with_(n_layers=6, dg_stride=2), 2, 517, [517, 200]),
    "depthgraft_full_map": (W["depthgraft"], 2, 130, [130, 65]),
    "peaky_hd128": (W["cla2_64k"].with_(n_layers=2), 2, 3000, [3000, 1777]),
    "mqa_g32_hd64": (W["tinyllama_cla2"].with_(n_layers=2, n_kv_heads=1), 2, 200, [200, 77]),
    "g16_hd128": (W["cla2_64k"].with_(n_layers=2, n_q_heads=16, n_kv_heads=1), 2, 333, [333, 64]),
    "g1_hd64": (W["tinyllama_cla2"].with_(n_layers=3, n_q_heads=4, n_kv_heads=4), 2, 150, [150, 99]),
    "g2_hd128_f32": (W["tiny_cla2"].with_(n_q_heads=4, head_dim=128), 2, 190, [190, 3]),
    "g8_hd128_mixed": (W["depthgraft"].with_(n_layers=6, dg_stride=2, n_q_heads=64), 1, 250, [250]),
    "g4_hd64_f32_mixed": (W["depthgraft"].with_(n_layers=6, dg_stride=2, head_dim=64, dtype="f32"), 2, 99, [99, 64]),
    # 64 sequences x 4 KV heads: a grid of 256 workgroups, where the hd-64 MFMA
    # decode runs three waves per workgroup (pages w, w+3, ...); ragged and
    # empty sequences
    "mfma_three_wave_grid": (W["tinyllama_cla2"].with_(n_layers=2), 64, 300,
                             [0, 1, 2, 63, 64, 65] + [(37 * i) % 300 + 1 for i in range(6, 63)] + [300]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_decode_matches_oracle(case):
    wl, B, ctx, lens = CASES[case]
    note(f"[decode parity] {case}: L={wl.n_layers} B={B} ctx={ctx} lens={lens} "
         f"Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} hd={wl.head_dim} {wl.dtype}")
    d = Dense(wl, B, ctx, lens)
    for l in range(wl.n_layers):
        got = d.decode(l)
        torch.cuda.synchronize()
        assert_close(got, d.oracle_decode(l), wl.dtype, f"{case} layer {l}")


def test_split_count_sweep_agrees():
    wl, B, ctx, lens = CASES["peaky_hd128"]
    d = Dense(wl, B, ctx, lens)
    ref = d.oracle_decode(1)
    n_pages = (ctx + 63) // 64
    outs = []
    for s in (1, 2, 7, n_pages, n_pages + 5):
        note(f"[split sweep] n_splits={s}")
        got = d.decode(1, n_splits=s)
        torch.cuda.synchronize()
        assert_close(got, ref, wl.dtype, f"n_splits={s}")
        outs.append(got.double().cpu())
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) < 2e-3


def test_three_wave_mfma_decode_across_split_counts():
    # grids of 256, 512 and 768 workgroups (S = 1, 2, 3): three waves for the
    # unsplit one, four for the others
    wl, B, ctx, lens = CASES["mfma_three_wave_grid"]
    d = Dense(wl, B, ctx, lens)
    ref = d.oracle_decode(1)
    for s in (1, 2, 3):
        note(f"[three-wave grid] n_splits={s}")
        got = d.decode(1, n_splits=s)
        torch.cuda.synchronize()
        assert_close(got, ref, wl.dtype, f"three-wave grid, n_splits={s}")


@pytest.mark.parametrize("name,wl,B,ctx", [
    # 32 query heads on one KV head (hd 64) and 16 on one (hd 128): the MFMA
    # decode with two 16-head blocks over one page load, and at hd 128
    ("g32_hd64", W["tinyllama_cla2"].with_(n_layers=2, n_kv_heads=1), 256, 130),
    ("g16_hd128", W["cla2_64k"].with_(n_layers=2, n_q_heads=16, n_kv_heads=1), 256, 130),
])
def test_large_group_mfma_decode(name, wl, B, ctx):
    lens = [ctx if i % 7 == 0 else (29 * i) % ctx + 1 for i in range(B)]
    lens[3] = 0
    d = Dense(wl, B, ctx, lens)
    ref = d.oracle_decode(1)
    # one partition: 256 workgroups of three waves; 2 and 3: four waves
    for s in (1, 2, 3):
        note(f"[large group] {name} n_splits={s}")
        got = d.decode(1, n_splits=s)
        torch.cuda.synchronize()
        assert_close(got, ref, wl.dtype, f"{name}, n_splits={s}")


def test_deterministic_and_page_permutation_invariant():
    wl, B, ctx, lens = CASES["tinyllama_shape_ragged"]
    d = Dense(wl, B, ctx, lens)
    a = d.decode(2)
    b = d.decode(2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    n_pages = B * ((ctx + 63) // 64)
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    dp = Dense(wl, B, ctx, lens, page_perm=perm)
    c = dp.decode(2)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_layers_sharing_a_source_are_bit_identical():
    wl, B, ctx, lens = CASES["tinyllama_shape_ragged"]
    d = Dense(wl, B, ctx, lens)
    q = d.q(0)
    a = d.decode(2, q=q)
    b = d.decode(3, q=q)
    c = d.decode(1, q=q)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_empty_and_single_key_sequences():
    wl = W["tinyllama_cla2"].with_(n_layers=2)
    d = Dense(wl, 3, 130, [0, 1, 130])
    got = d.decode(1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(got[0]) == 0
    g = wl.group
    v0 = d.v[0][1, 0].double()                      # [Hkv, hd] of the only key
    want = v0.repeat_interleave(g, dim=0)
    assert float((got[1].double().cpu() - want).abs().max()) < 1e-6
    assert_close(got, d.oracle_decode(1), "bf16", "empty/single")


def test_bf16_output():
    wl, B, ctx, lens = CASES["peaky_hd128"]
    d = Dense(wl, B, ctx, lens)
    got = d.decode(0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = d.oracle_decode(0)
    err = np.abs(got.double().cpu().numpy() - ref)
    assert np.all(err <= TOL_ABS + 2.0 ** -8 * np.abs(ref))


def _page_offset(layout_pt, b, pos, kvh, hd, Hkv, n_phys, slot):
    page = int(layout_pt[b, pos // 64])
    return ((slot * n_phys + page) * Hkv + kvh) * 64 * hd


def test_append_layout_bit_exact_and_incremental():
    """Bulk append vs token-by-token appends give identical pools, and the
    pool bytes sit where the documented page layouts put them."""
    wl = W["tinyllama_cla2"].with_(n_layers=2, n_q_heads=8, n_kv_heads=2)
    B, ctx = 2, 140
    bulk = Dense(wl, B, ctx, [ctx, ctx], nan_fill="zero")
    inc = Dense(wl, B, ctx, [ctx, ctx], nan_fill="zero", append_lens=[0, 0])
    k, v = bulk.k[0].cuda(), bulk.v[0].cuda()
    bulk_k = bulk.cache.k_pool.clone()
    for t in range(ctx):
        sp = torch.full((B,), t, dtype=torch.int32, device="cuda")
        K.kvs_append(inc.plan, inc.cache, 0, k[:, t:t + 1].contiguous(), v[:, t:t + 1].contiguous(), sp)
    torch.cuda.synchronize()
    assert torch.equal(inc.cache.k_pool, bulk_k)
    assert torch.equal(inc.cache.v_pool, bulk.cache.v_pool)
    # layout formula
    kp = bulk.cache.k_pool.view(torch.bfloat16).cpu()
    vp = bulk.cache.v_pool.view(torch.bfloat16).cpu()
    pt = bulk.cache.page_table.cpu()
    hd, Hkv, n_phys = 64, 2, bulk.cache.sizes.n_phys_pages
    for b in range(B):
        for pos in (0, 1, 63, 64, 101, 139):
            for kvh in range(Hkv):
                base = _page_offset(pt, b, pos, kvh, hd, Hkv, n_phys, 0)
                t = pos % 64
                E, ncw = 8, hd // 64

                def koff(d):
                    c = d // E
                    return (((t // 8) * ncw + c // 8) * 64 + 8 * (t % 8) + c % 8) * E + d % E

                krow = torch.stack([kp[base + koff(d)] for d in range(hd)])
                vrow = torch.stack([vp[base + (t // 2) * hd * 2 + d * 2 + t % 2] for d in range(hd)])
                assert torch.equal(krow, bulk.k[0][b, pos, kvh])
                assert torch.equal(vrow, bulk.v[0][b, pos, kvh])


@pytest.mark.parametrize("name,layers,sample_b", [
    ("tinyllama_cla2", [0, 1], [0, 37, 63]),
    ("depthgraft", None, [0, 7]),
    ("cla2_64k", [0, 1], [0, 3]),
])
def test_full_size_sampled(name, layers, sample_b):
    """Workload shapes at full size, library's own split choice (the bench's
    launch configuration); the oracle checks every head of sampled sequences."""
    wl = W[name]
    if name == "depthgraft":
        # a 24-layer map needs 16 owner slots; keep layer 16 (reads 8 and 0)
        # and its sources by trimming the map to 17 layers
        wl = wl.with_(n_layers=17)
        layers = [8, 16]
    else:
        wl = wl.with_(n_layers=2)
    note(f"[full size] {name}: B={wl.batch} ctx={wl.ctx} layers={layers}")
    d = Dense(wl, wl.batch, wl.ctx, [wl.ctx] * wl.batch, kv_device="cuda", nan_fill=False)
    for l in layers:
        q = d.q(l)
        got = d.decode(l, q=q).double().cpu()
        torch.cuda.synchronize()
        for b in sample_b:
            kk = {s: d.k[s][b:b + 1] for s in d.k}
            vv = {s: d.v[s][b:b + 1] for s in d.v}
            ref = A.layer_decode(d.src.tolist(), d.w.tolist(), l, kk, vv, q[b:b + 1], [wl.ctx])
            max_abs, rel = errors(got[b:b + 1], ref)
            note(f"   layer {l} b {b}: max_abs {max_abs:.2e} rel {rel:.2e}")
            assert max_abs <= 1e-2 and rel <= 5e-3


def test_timed_launch_events_bracket_the_kernel():
    """kvs_time_next_launch: the armed call's output is the unarmed call's, its
    kernel events give a positive duration no longer than the whole call, and
    the arming is consumed by one call (the next call leaves the events alone)."""
    wl, B, ctx, lens = CASES["peaky_hd128"]
    note("[timed launch] decode with kernel events, S = 4")
    d = Dense(wl, B, ctx, lens)
    ref = d.decode(0, n_splits=4)
    e0, e1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    K.kvs_time_next_launch(k0, k1)
    e0.record()
    got = d.decode(0, n_splits=4)
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    kernel_ms, call_ms = k0.elapsed_time(k1), e0.elapsed_time(e1)
    assert 0.0 < kernel_ms <= call_ms
    stamp = k1.elapsed_time(k0)
    d.decode(0, n_splits=4)            # not armed: k0, k1 keep their timestamps
    torch.cuda.synchronize()
    assert k1.elapsed_time(k0) == stamp
