"""Shared-KV decode attention benchmark on one MI355X.

A step is one decode step of the whole hot path over all layers of the
workload: every owner layer appends its new token's K/V (kvs_append, n=1),
then every layer runs split-K decode attention over its source slot(s)
(kvs_attn_decode: the partition kernel, plus a small merge kernel when the
sequence is split into several partitions).  The factorized workload
appends the new token's coefficients, codes, scales and rank
(kvs_append_factorized) instead of K/V.  Inputs are resident in HBM before
the timed region; K/V and queries are seeded synthetic N(0,1) tensors of
the workload's shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--roofline-only] [--no-cpu-baseline] [--no-extras]
    python bench.py --sweep [--sweep-out FILE]

The default workload is the long-context decode: 32 layers, CLA2 map, batch
4, context 65536, 32 q / 8 KV heads, head_dim 128, bf16, 1% of keys x4.
Prints one JSON line.  ``value`` is decode tokens/s (one token per sequence
per step, warm back-to-back steps); ``ms_per_step_cold`` is the same step
with the 256 MB Infinity Cache flushed before every layer's calls (the
flush itself outside the timed intervals).  ``roofline`` rates the decode
launch of a single-source layer against the 8 TB/s HBM peak with its
algorithmic bytes (every source tile, K and V, read once): its duration is
timed with a pair of HIP events that the library attaches to the decode
kernel's own start and end (kvs_time_next_launch, i.e. hipExtLaunchKernel;
the partition merge and the launch latency are reported apart as
avg_call_us), with the cache flushed before each launch by reading a 512 MB
buffer (a read leaves no dirty lines whose write-back would compete with
the timed launch), so no byte of the timed launch is served from a cache.
``cpu_baseline`` times the fp64 oracle (one BLAS thread) on a bounded
sample of the same workload, scaled to the metric's unit.  The default run
adds the 64K factorized decode (``roofline_factorized``, with its own CPU
baseline) and the 4-layer fp32 toy step's time (``tiny_cla2``).

``--sweep`` times the metric's batch x context grid: the 1.1B-shaped CLA2
decode at B in {1, 8, 16, 32, 64, 128} x ctx in {512, 1024, 2048} and the
long-context CLA2 decode at B in {1, 2, 4, 8} x ctx in {16K, 32K, 64K}:
tokens/s and HBM rates of the warm step, the cold step and the cache-flushed
kernel; one JSON line, and a markdown table with --sweep-out.
"""
import argparse
import gc
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attention_cross_layer_amd as K  # noqa: E402
import datagen  # noqa: E402

METRIC = "shared-KV decode attn: tokens/s and achieved HBM GB/s (% of peak) per batch x ctx"
HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20
DEFAULT_WORKLOAD = "cla2_64k"
CPU_BUDGET_S = 12.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def describe(wl, src):
    owners = datagen.owner_layers(src)
    mixed = sum(1 for l in range(wl.n_layers) if int(src[l, 1]) >= 0)
    return {"workload": wl.name, "layers": wl.n_layers, "owner_layers": len(owners),
            "mixed_layers": mixed, "batch": wl.batch, "ctx": wl.ctx, "q_heads": wl.n_q_heads,
            "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "share": wl.share,
            "peaky_frac": wl.peaky_frac}


def bytes_per_call(wl, src, l):
    """Algorithmic bytes of one decode call of layer l: every source tile (K and
    V) read once; queries and outputs (< 0.5%) not counted."""
    elem = 4 if wl.dtype == "f32" else 2
    per_source = wl.batch * wl.n_kv_heads * wl.ctx * wl.head_dim * 2 * elem
    return per_source * (1 if int(src[l, 1]) < 0 else 2)


def setup(wl):
    src, w = datagen.share_map(wl)
    cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.dtype,
                        wl.batch, wl.ctx)
    plan = K.kvs_share_plan(cfg, src, w)
    cache = K.Cache(plan, "cuda")
    owners = datagen.owner_layers(src)
    zeros = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    for l in owners:
        k, v = datagen.owner_kv(wl, l, device="cuda")
        K.kvs_append(plan, cache, l, k, v, zeros)
        del k, v
    torch.cuda.synchronize()
    return src, w, plan, cache, owners


def setup_factorized(wl):
    """Factorized cache: every layer pair's coefficients and bases, every
    layer's int8 residual codes, scales and directions, per-token ranks."""
    src, w = datagen.share_map(wl)
    cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", wl.batch,
                        wl.ctx, kind=K.KVS_FACTORIZED, basis_rank=wl.basis_rank,
                        resid_rank_max=wl.resid_rank_max)
    plan = K.kvs_share_plan(cfg, src, w)
    cache = K.Cache(plan, "cuda")
    owners = datagen.owner_layers(src)
    Hkv, R, Rm, hd = wl.n_kv_heads, wl.basis_rank, wl.resid_rank_max, wl.head_dim
    rank = datagen.token_ranks(wl, device="cuda")
    bk_all = cache.basis_k.view(torch.bfloat16).view(len(owners), Hkv, R, hd)
    bv_all = cache.basis_v.view(torch.bfloat16).view(len(owners), Hkv, R, hd)
    uk_all = cache.ubasis_k.view(torch.bfloat16).view(wl.n_layers, Hkv, Rm, hd)
    uv_all = cache.ubasis_v.view(torch.bfloat16).view(wl.n_layers, Hkv, Rm, hd)
    zeros = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    for l in range(wl.n_layers):
        ck = cv = None
        if l in owners:
            ck, cv = datagen.pair_coeffs(wl, l // 2, device="cuda")
            bk, bv = datagen.pair_basis(wl, l // 2, device="cuda")
            bk_all[owners.index(l)].copy_(bk)
            bv_all[owners.index(l)].copy_(bv)
        uk, uv = datagen.layer_residual_basis(wl, l, device="cuda")
        uk_all[l].copy_(uk)
        uv_all[l].copy_(uv)
        dk, dv, sk, sv = datagen.layer_residual(wl, l, rank, device="cuda")
        K.kvs_append_factorized(plan, cache, l, ck, cv, dk, dv, sk, sv, rank, zeros)
    torch.cuda.synchronize()
    return src, w, plan, cache, owners, rank


def fact_bytes_per_call(wl, rank):
    """Algorithmic bytes of one factorized decode call: per (sequence, KV head,
    token) both coefficient rows (2 x 32 bf16), r_t int8 codes for K and for
    V, two fp16 scales; one rank byte per (sequence, token)."""
    tokens = wl.batch * wl.ctx
    sum_r = int(rank.to(torch.int64).sum())
    return wl.n_kv_heads * (tokens * (2 * wl.basis_rank * 2 + 4) + 2 * sum_r) + tokens



# ----------------------------------------------------------------------------
# the oracle timed on the host: one BLAS thread, a bounded sample of the
# workload's units, inputs prepared outside the timed region, the oracle's
# own bf16/fp16/int8 -> fp64 upcast inside it
# ----------------------------------------------------------------------------

def oracle_time(prep, run, budget_s):
    """Call run(*prep(i)) for i = 0, 1, ... until ``budget_s`` seconds of
    timed run() calls; returns (calls, seconds)."""
    from threadpoolctl import threadpool_limits

    done, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            args = prep(done)
            t0 = time.perf_counter()
            run(*args)
            elapsed += time.perf_counter() - t0
            done += 1
    return done, elapsed


def cpu_dense_decode(rig, budget_s=CPU_BUDGET_S):
    """Oracle decode of whole layer calls of one sequence after another
    (layers in order, then the next sequence): effective K/V of the layer's
    sources, then attention over every key.  Rate in tokens/s = sequence
    steps (L layer calls each) per second."""
    from oracle import attention as A

    wl, L = rig.wl, rig.wl.n_layers
    src, w = rig.src.tolist(), rig.w.tolist()
    host, cur = {}, [-1]

    def prep(i):
        b, l = (i // L) % wl.batch, i % L
        if b != cur[0]:
            host.clear()
            cur[0] = b
        for s in (int(x) for x in rig.src[l] if int(x) >= 0):
            if s not in host:
                k, v = datagen.owner_kv(wl, s, device="cuda")
                k[:, wl.ctx - 1:] = rig.new_kv[s][0]
                v[:, wl.ctx - 1:] = rig.new_kv[s][1]
                host[s] = (k[b:b + 1].cpu(), v[b:b + 1].cpu())
                del k, v
        return l, rig.qs[l][b:b + 1].cpu()

    def run(l, q):
        A.layer_decode(src, w, l, {s: kv[0] for s, kv in host.items()},
                       {s: kv[1] for s, kv in host.items()}, q, [wl.ctx])

    done, el = oracle_time(prep, run, budget_s)
    return {"value": done / L / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} layer calls ({done / L:.2f} sequence decode steps of {L} layers) at "
                      f"ctx {wl.ctx}, sequences taken in turn, {el:.1f} s; rate = sequence steps/s; "
                      f"bf16->fp64 upcast included"}


def cpu_fact_decode(rig, budget_s=CPU_BUDGET_S):
    """Oracle decode over the factorized cache: every key and value of the
    layer rebuilt from its coefficients, basis, scaled codes and residual
    directions (the plain definition), then attention; layer calls of one
    sequence after another."""
    from oracle import attention as A

    wl, L = rig.wl, rig.wl.n_layers
    T = wl.ctx
    one_b = {}

    def host_layer(b, l):
        o = int(rig.src[l, 0])
        ck, cv = datagen.pair_coeffs(wl, o // 2, device="cuda")
        bk, bv = datagen.pair_basis(wl, o // 2, device="cuda")
        uk, uv = datagen.layer_residual_basis(wl, l, device="cuda")
        dk, dv, sk, sv = datagen.layer_residual(wl, l, rig.rank, device="cuda")
        nf_o, nf_l = rig.new_f[o], rig.new_f[l]
        ck[:, T - 1:], cv[:, T - 1:] = nf_o[0], nf_o[1]
        dk[:, T - 1:], dv[:, T - 1:], sk[:, T - 1:], sv[:, T - 1:] = nf_l[2], nf_l[3], nf_l[4], nf_l[5]
        sl = slice(b, b + 1)
        return tuple(x[sl].cpu() for x in (ck, cv, dk, dv, sk, sv)) + (
            bk.cpu(), bv.cpu(), uk.cpu(), uv.cpu(), rig.rank[sl].cpu())

    def prep(i):
        b, l = (i // L) % wl.batch, i % L
        one_b.clear()
        one_b["x"] = host_layer(b, l)
        return l, rig.qs[l][b:b + 1].cpu()

    def run(l, q):
        ck, cv, dk, dv, sk, sv, bk, bv, uk, uv, r = one_b["x"]
        kk = A.factorized_kv(ck, bk, sk, dk, uk, r)
        vv = A.factorized_kv(cv, bv, sv, dv, uv, r)
        A.attend_decode(q, kk, vv, [T])

    done, el = oracle_time(prep, run, budget_s)
    return {"value": done / L / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} layer calls ({done / L:.2f} sequence decode steps of {L} layers) at "
                      f"ctx {T}: every key/value rebuilt from the factorized entries, then "
                      f"attention, {el:.1f} s; rate = sequence steps/s"}


def cpu_prefill(wl, layers, host_kv, qs, n, budget_s=CPU_BUDGET_S):
    """Oracle causal prefill chunk, one (layer, query head) at a time: that
    head's n queries over the keys of its KV head.  The step time is the
    mean time per (layer, head) times heads x layers."""
    from oracle import attention as A

    G, T, Hq = wl.group, wl.ctx, wl.n_q_heads
    units = [(l, h) for l in layers for h in range(Hq)]

    def prep(i):
        l, h = units[i % len(units)]
        k, v = host_kv(l)
        g = h // G
        return qs[l][:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1]

    def run(q, k, v):
        A.attend_prefill(q, k, v, [T], causal=True)

    done, el = oracle_time(prep, run, budget_s)
    step_s = el / done * Hq * len(layers)
    return {"value": n / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (layer, query head) units of the {n}-query causal chunk over {T} keys "
                      f"in {el:.1f} s, scaled by {Hq} heads x {len(layers)} layers "
                      f"= {Hq * len(layers) / done:.1f}x the timed sample"}


def cpu_fact_prefill(wl, layers, host_layer, qs, n, budget_s=CPU_BUDGET_S):
    """Oracle causal prefill over the factorized cache, one (layer, KV head)
    at a time: that head's keys and values rebuilt from the factorized
    entries, then the G query heads' chunk attention over them."""
    from oracle import attention as A

    G, T, Hkv = wl.group, wl.ctx, wl.n_kv_heads
    units = [(l, g) for l in layers for g in range(Hkv)]

    def prep(i):
        l, g = units[i % len(units)]
        ck, cv, dk, dv, sk, sv, bk, bv, uk, uv, r = host_layer(l)
        hs = slice(g, g + 1)
        return (l, g, ck[:, :, hs], cv[:, :, hs], dk[:, :, hs], dv[:, :, hs], sk[:, :, hs],
                sv[:, :, hs], bk[hs], bv[hs], uk[hs], uv[hs], r)

    def run(l, g, ck, cv, dk, dv, sk, sv, bk, bv, uk, uv, r):
        kk = A.factorized_kv(ck, bk, sk, dk, uk, r)
        vv = A.factorized_kv(cv, bv, sv, dv, uv, r)
        for h in range(g * G, (g + 1) * G):
            A.attend_prefill(qs[l][:, :, h:h + 1], kk, vv, [T], causal=True)

    done, el = oracle_time(prep, run, budget_s)
    step_s = el / done * Hkv * len(layers)
    return {"value": n / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (layer, KV head) units (rebuild of that head's {T} keys/values, then "
                      f"its {G} query heads' {n}-query causal chunk) in {el:.1f} s, scaled by "
                      f"{Hkv} KV heads x {len(layers)} layers = {Hkv * len(layers) / done:.1f}x"}


def cpu_encode(wl, n, rows, owner_of, bases, rank, budget_s=CPU_BUDGET_S):
    """Oracle encoder over whole layers: coefficients from the slot owner's
    rows, residual coordinates on the layer's directions, fp16 scale and
    int8 codes at each token's rank, for K and V."""
    from oracle import factorize as F

    L = wl.n_layers

    def prep(i):
        l = i % L
        o = owner_of(l)
        bk, bv, uk, uv = bases(l)
        return (rows[l][0].cpu(), rows[o][0].cpu(), rows[l][1].cpu(), rows[o][1].cpu(),
                bk.cpu(), bv.cpu(), uk.cpu(), uv.cpu(), rank.cpu())

    def run(k, ko, v, vo, bk, bv, uk, uv, r):
        F.encode(k, ko, bk, uk, r)
        F.encode(v, vo, bv, uv, r)

    done, el = oracle_time(prep, run, budget_s)
    step_s = el / done * L
    return {"value": n / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} layers of the {n}-token chunk encoded (K and V) in {el:.1f} s, "
                      f"scaled to {L} layers ({L / done:.1f}x the timed sample)"}




MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_WORKLOAD = "depthgraft_prefill_chunk"
FACT_PREFILL_WORKLOAD = "factorized_prefill_chunk"
PREFILL_WORKLOADS = (PREFILL_WORKLOAD, FACT_PREFILL_WORKLOAD)
ENCODE_WORKLOAD = "factorized_encode_chunk"
CALIB_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"decode_kernel": "k_decode.hip", "decode_mfma_kernel": "k_decode.hip",
                  "fact_decode_kernel": "k_factorized.hip",
                  "prefill_kernel": "k_prefill.hip", "fact_prefill_kernel": "k_fact_prefill.hip",
                  "encode_kernel": "k_encode.hip"}


def source_digest(kernel):
    import hashlib
    path = os.path.join(ROOT, "attention_cross_layer_amd", "csrc",
                        KERNEL_SOURCES[kernel.split("<")[0]])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per launch measured by the committed counter profile of this
    workload's dominant kernel, or None when there is none or the kernel's
    source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE)).get(workload)
    if not rec or rec["source_sha256_16"] != source_digest(rec["kernel"]):
        return None
    return {"bytes_per_launch": rec["fetch_bytes"] + rec["write_bytes"],
            "source": f"rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated ({rec['profile']})"}


def summarize(prof_dir, kernel, workload):
    """Summarise a profile directory holding kt/ (--kernel-trace --stats),
    fetch/ (--pmc FETCH_SIZE) and write/ (--pmc WRITE_SIZE) runs of
    ``bench.py --roofline-only``: average duration of ``kernel`` and its
    counter bytes per dispatch, scaled by what the same counters read for the
    run's 256 MiB reference copy."""
    import csv
    import glob

    def rows(sub, name):
        f = glob.glob(os.path.join(prof_dir, sub, "*" + name))
        return list(csv.DictReader(open(f[0]))) if f else []

    # ``kernel`` is a kernel name (every instantiation) or one instantiation,
    # e.g. "decode_kernel<unsigned short, 128, 4, 1>"
    key = "::" + kernel + ("" if "<" in kernel else "<")

    def match(name):
        return key in name

    stats = [r for r in rows("kt", "kernel_stats.csv") if match(r["Name"])]
    out = {"kernel": kernel, "workload": workload}
    if stats:
        calls = sum(int(r["Calls"]) for r in stats)
        tot = sum(float(r["TotalDurationNs"]) for r in stats)
        out |= {"calls": calls, "avg_us": tot / calls / 1e3}
    for sub, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        rs = [r for r in rows(sub, "counter_collection.csv") if r["Counter_Name"] == counter]
        mine = [float(r["Counter_Value"]) for r in rs if match(r["Kernel_Name"])]
        # the reference copy is the run's last device-to-device copy dispatch
        copy = [float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"]]
        if mine and copy:
            scale = CALIB_BYTES / (copy[-1] * 1024)      # bytes per counted byte
            out[counter] = {"kib_per_dispatch": sum(mine) / len(mine),
                            "copy_kib": copy[-1], "scale": scale,
                            "bytes_per_dispatch": sum(mine) / len(mine) * 1024 * scale}
    return out


def algorithmic_bytes(wl, kernel):
    """Algorithmic bytes of one launch of the profiled kernel: a dense decode
    launch of a layer with as many sources as the instantiation's last
    template argument (one when the name carries none), or a factorized
    decode launch."""
    if kernel.startswith("fact_decode_kernel"):
        B, T = wl.batch, wl.ctx
        n_hi = int(round(wl.rank16_frac * T))
        sum_r = B * (16 * n_hi + 8 * ((T - n_hi) // 2))   # exact per-rank token counts
        tokens = B * T
        return wl.n_kv_heads * (tokens * (2 * wl.basis_rank * 2 + 4) + 2 * sum_r) + tokens
    if kernel.startswith("fact_prefill_kernel"):
        # queries in, outputs out (bf16), every coefficient row, code, scale
        # and meta entry of the sequence once
        n, T = wl.prefill_n, wl.ctx
        n_hi = int(round(wl.rank16_frac * T))
        sum_r = 16 * n_hi + 8 * ((T - n_hi) // 2)
        return (n * wl.n_q_heads * wl.head_dim * 2 * 2
                + wl.n_kv_heads * (T * (2 * wl.basis_rank * 2 + 4) + 2 * sum_r) + 2 * T)
    if kernel.startswith("prefill_kernel"):
        # queries in, outputs out (bf16), every K/V tile of the sequence once
        n, T = wl.prefill_n, wl.ctx
        return (n * wl.n_q_heads * wl.head_dim * 2 * 2
                + wl.batch * T * wl.n_kv_heads * wl.head_dim * 2 * 2)
    nsrc = (int(kernel.rstrip(">").split(",")[-1])
            if "<" in kernel and kernel.startswith("decode_kernel") else 1)
    elem = 4 if wl.dtype == "f32" else 2
    return wl.batch * wl.n_kv_heads * wl.ctx * wl.head_dim * 2 * elem * nsrc


def record_profile(prof_dir, kernel, workload, s):
    """Write profiles/<kernel>_<workload>.md from a summarised profile
    directory and store its counter bytes in profiles/traffic.json."""
    import csv
    import glob

    prefill = workload in PREFILL_WORKLOADS
    wl = prefill_wl(workload) if prefill else datagen.WORKLOADS[workload]
    base = kernel.split("<")[0]
    f = glob.glob(os.path.join(prof_dir, "kt", "*kernel_stats.csv"))
    allk = sorted(csv.DictReader(open(f[0])), key=lambda r: -float(r["TotalDurationNs"]))
    top = [r for r in allk if "kvs::" in r["Name"]] + [r for r in allk if "kvs::" not in r["Name"]][:4]
    alg = algorithmic_bytes(wl, kernel)
    fetch, write = s["FETCH_SIZE"]["bytes_per_dispatch"], s["WRITE_SIZE"]["bytes_per_dispatch"]
    cmd = (f"python3 bench.py --workload {workload} --steps 8 --warmup 2 --no-cpu-baseline" if prefill
           else f"python3 bench.py --workload {workload} --roofline-only")
    lines = [
        f"# `{kernel}` on `{workload}`", "",
        "Commands (from the repository root, profile directory `P`):", "", "```",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d P/kt -o run -- {cmd}",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d P/fetch -o run -- {cmd}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d P/write -o run -- {cmd}",
        f"python3 bench.py --summarize P --kernel '{kernel}' --workload {workload} --record",
        "```", "",
        f"Kernel source sha256[:16]: `{s['source_sha256_16']}`", "",
        f"## `{kernel}`", "",
        f"- dispatches: {s['calls']}, average duration {s['avg_us']:.2f} us",
        f"- algorithmic bytes per launch: {alg:,}",
        f"- FETCH_SIZE: {s['FETCH_SIZE']['kib_per_dispatch']:.1f} KiB/dispatch x "
        f"{s['FETCH_SIZE']['scale']:.4f} (copy calibration: 256 MiB read counted as "
        f"{s['FETCH_SIZE']['copy_kib']:.1f} KiB) = {fetch:,.0f} B "
        f"({fetch / alg:.3f} x the algorithmic bytes"
        + (", which count reads and writes)" if prefill else ")"),
        f"- WRITE_SIZE: {s['WRITE_SIZE']['kib_per_dispatch']:.1f} KiB/dispatch x "
        f"{s['WRITE_SIZE']['scale']:.4f} = {write:,.0f} B"
        + (f"; read + written = {(fetch + write) / alg:.3f} x algorithmic" if prefill else ""),
        (f"- algorithmic MFMA rate at the traced average: "
         f"{prefill_kernel_flops(wl, kernel) / (s['avg_us'] * 1e-6) / 1e12:,.0f}"
         f" TFLOP/s ({prefill_kernel_flops(wl, kernel) / (s['avg_us'] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS:.1%}"
         f" of 2.5 PFLOP/s bf16; the profiler slows this launch)" if prefill else
         f"- algorithmic rate at the traced average: {alg / (s['avg_us'] * 1e-6) / 1e9:,.0f} GB/s "
         f"({alg / (s['avg_us'] * 1e-6) / 1e9 / HBM_PEAK_GBS:.1%} of 8 TB/s)"), "",
        "## Kernels of the traced run: this library's, then the largest others (set-up, "
        "and the 512 MB read that flushes the cache before each timed launch)", "",
        "| kernel | calls | avg us | share |", "|---|---:|---:|---:|"]
    for r in top:
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
        name = name.replace("void ", "").replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    out = os.path.join(ROOT, "profiles", f"{base}_{workload}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    rec = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    rec[workload] = {"kernel": kernel, "source_sha256_16": s["source_sha256_16"],
                     "fetch_bytes": round(fetch), "write_bytes": round(write),
                     "algorithmic_bytes": alg, "avg_us": s["avg_us"],
                     "profile": os.path.relpath(out, ROOT)}
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    return out


def calibration_copy():
    """Reference copy of known size for calibrating the HBM byte counters of a
    profiled run: 256 MiB read + 256 MiB written by PyTorch's elementwise
    copy kernel, cache flushed first (the run's last device copy)."""
    flush = torch.ones((FLUSH_BYTES // 4 // 4096, 4096), dtype=torch.float32, device="cuda")
    ref_src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    ref_dst = torch.empty_like(ref_src)
    flush.sum(dim=0)
    ref_dst.copy_(ref_src)
    torch.cuda.synchronize()


def decode_kernel_name(wl, two_source):
    """The kernel a decode call of this workload launches for its partitions."""
    G = wl.n_q_heads // wl.n_kv_heads
    if wl.dtype == "bf16" and not two_source and ((wl.head_dim == 64 and G <= 32)
                                                  or (wl.head_dim == 128 and G == 16)):
        return "decode_mfma_kernel (bf16 MFMA, split-K partitions)"
    return "decode_kernel (split-K partitions)"


def prefill_flops(n, T, n_q_heads, hd):
    """Algorithmic FLOPs of a causal chunk: only unmasked (query, key) pairs,
    QK^T and PV each 2*hd per pair."""
    pairs = n * (T - n) + n * (n + 1) // 2
    return pairs * 4 * hd * n_q_heads


def fact_prefill_flops(n, T, n_q_heads, hd, width=48):
    """Algorithmic FLOPs of a causal chunk over the factorized cache in the
    coefficient space: per unmasked (query, key) pair 2*width for the score
    and 2*width for the value accumulation (width = basis rank + residual
    rank bound); per query row 2*hd*width to project it onto the bases and
    2*hd*width to map its accumulators back."""
    pairs = n * (T - n) + n * (n + 1) // 2
    return n_q_heads * (pairs * 4 * width + n * 4 * hd * width)


def prefill_wl(workload):
    """Workload of a prefill benchmark: the DepthGraft chunk (4096 queries at
    offset 4096 of an 8192-token prompt, batch 1) or the same chunk on the
    64K factorized model's shape."""
    if workload == FACT_PREFILL_WORKLOAD:
        return datagen.WORKLOADS["factorized_64k"].with_(batch=1, ctx=8192, prefill_n=4096,
                                                         prefill_batch=1)
    return datagen.WORKLOADS["depthgraft"].with_(batch=1)


FP32_VECTOR_PEAK_TFLOPS = 157.3
# VALU lane-operations an unmasked (query, key) pair needs in an online
# softmax whose probabilities feed a bf16 product: one fma (scale and
# shift), one exp2 (a transcendental: a quarter of the fma rate, so four fma
# slots), and half of a max3, a pack to bf16 and a dot2 into the running sum
# (each covers two pairs).
VALU_SLOTS_PER_PAIR = 1 + 4 + 3 * 0.5


def issue_roofline(wl, fact, us):
    """The prefill chunk against what issuing its instructions allows: the
    softmax's VALU work per pair at the fp32 vector rate plus the MFMA work
    per pair as the kernel issues it, the two not overlapped (per-SIMD issue
    counters show them serialised).  MFMA FLOPs issued per pair: dense
    4*hd (two products); factorized 2*(R + Rmax) for the scores (q~, u~ as
    fp16, one product) + 2*(R + 2*Rmax) for the values (the
    residual product runs 32 rows wide, half of them zero)."""
    n, T = wl.prefill_n, wl.ctx
    pairs = wl.n_q_heads * (n * (T - n) + n * (n + 1) // 2)
    R, Rm = wl.basis_rank, wl.resid_rank_max
    mfma_flops = (2 * (R + Rm) + 2 * (R + 2 * Rm)) if fact else 4 * wl.head_dim
    valu_s = VALU_SLOTS_PER_PAIR / (FP32_VECTOR_PEAK_TFLOPS * 1e12 / 2)
    mfma_s = mfma_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    peak = 1.0 / (valu_s + mfma_s)
    achieved = pairs / (us * 1e-6)
    return {"bound": "alu", "unit": "pairs/s", "achieved": achieved, "peak": peak,
            "frac": achieved / peak, "valu_slots_per_pair": VALU_SLOTS_PER_PAIR,
            "mfma_flops_per_pair_issued": mfma_flops,
            "note": "softmax VALU at the fp32 vector rate + issued MFMA at the bf16 rate, serialised"}


def prefill_kernel_flops(wl, kernel):
    if kernel.startswith("fact_prefill_kernel"):
        return fact_prefill_flops(wl.prefill_n, wl.ctx, wl.n_q_heads, wl.head_dim,
                                  wl.basis_rank + wl.resid_rank_max)
    return prefill_flops(wl.prefill_n, wl.ctx, wl.n_q_heads, wl.head_dim)




def prefill_main(args, workload):
    """Prefill-chunk attention over one chunk per layer that needs it.

    depthgraft_prefill_chunk: the second 4096-token chunk of an 8192-token
    prompt (queries at 4096..8191, causal), batch 1, over the 16 owner layers
    of the DepthGraft map (the deeper layers own no cache entries, so prompt
    tokens need not run them); a step appends the chunk's K/V to each owner
    layer and runs its prefill-chunk attention.
    factorized_prefill_chunk: the same chunk on the 64K factorized model's
    shape (32 layers in 16 pairs, 32 q / 8 KV heads, hd 128, basis rank 32,
    residual ranks 0/8/16); a step appends the chunk's factorized entries
    (pair coefficients from the owner layer, each layer's codes and scales)
    and runs every layer's prefill-chunk attention."""
    if args.gpus != 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        sys.exit(2)
    fact = workload == FACT_PREFILL_WORKLOAD
    wl = prefill_wl(workload)
    n, T = wl.prefill_n, wl.ctx
    torch.cuda.set_device(0)
    log(f"[bench] setting up {workload}: {wl.name} prefill chunk n={n} at offset {T - n}")
    start = torch.full((1,), T - n, dtype=torch.int32, device="cuda")
    seq_len = torch.full((1,), T, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    if fact:
        src, w, plan, cache, owners, rank = setup_factorized(wl)
        layers = list(range(wl.n_layers))
        r_chunk = rank[:, T - n:].contiguous()
        chunk = {}
        for l in layers:
            cc = (tuple(x[:, T - n:].contiguous() for x in datagen.pair_coeffs(wl, l // 2, device="cuda"))
                  if l in owners else (None, None))
            res = tuple(x[:, T - n:].contiguous()
                        for x in datagen.layer_residual(wl, l, rank, device="cuda"))
            chunk[l] = cc + res

        def append(l):
            ck, cv, dk, dv, sk, sv = chunk[l]
            K.kvs_append_factorized(plan, cache, l, ck, cv, dk, dv, sk, sv, r_chunk, start,
                                    stream=stream)
        flops = fact_prefill_flops(n, T, wl.n_q_heads, wl.head_dim, wl.basis_rank + wl.resid_rank_max)
        kernel = "fact_prefill_kernel (fp16 score / bf16 value MFMA in the coefficient space, causal)"
    else:
        src, w, plan, cache, owners = setup(wl)
        layers = owners
        chunk = {l: datagen.owner_kv(wl, l, device="cuda") for l in owners}
        chunk = {l: (kv[0][:, T - n:].contiguous(), kv[1][:, T - n:].contiguous())
                 for l, kv in chunk.items()}

        def append(l):
            K.kvs_append(plan, cache, l, chunk[l][0], chunk[l][1], start, stream=stream)
        flops = prefill_flops(n, T, wl.n_q_heads, wl.head_dim)
        kernel = "prefill_kernel (bf16 MFMA, causal)"
    qs = {l: datagen.prefill_q(wl, l, n, device="cuda") for l in layers}
    outs = {l: torch.empty((1, n, wl.n_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
            for l in layers}
    ev = {l: [] for l in layers}

    def step(record=False):
        for l in layers:
            append(l)
            if record:
                e0, e1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
                K.kvs_time_next_launch(k0, k1, stream)
                e0.record(stream)
            K.kvs_attn_prefill_chunk(plan, cache, l, qs[l], seq_len, causal=True, out=outs[l],
                                     stream=stream)
            if record:
                e1.record(stream)
                ev[l].append((e0, e1, k0, k1))

    for _ in range(args.warmup):
        step()
    # the timed launch path's first use sets it up: once, outside the timing
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    K.kvs_time_next_launch(w0, w1, stream)
    K.kvs_attn_prefill_chunk(plan, cache, layers[0], qs[layers[0]], seq_len, causal=True,
                             out=outs[layers[0]], stream=stream)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step(record=True)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    n_calls = args.steps * len(layers)
    us = sum(k0.elapsed_time(k1) for l in layers for (e0, e1, k0, k1) in ev[l]) * 1e3 / n_calls
    call_us = sum(e0.elapsed_time(e1) for l in layers for (e0, e1, k0, k1) in ev[l]) * 1e3 / n_calls
    achieved = flops / (us * 1e-6) / 1e12
    res = {"metric": "shared-KV prefill chunk attn: prefill tokens/s and MFMA utilisation",
           "value": n * 1000.0 / ms, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": workload, "layers": len(layers),
                      "batch": 1, "chunk": n, "ctx": T, "causal": True,
                      "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                      "head_dim": wl.head_dim},
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                        "traffic": None, "kernel": kernel,
                        "flops_per_launch": flops, "avg_launch_us": us,
                        "timing": "HIP events on the kernel's own start and end (hipExtLaunchKernel)",
                        "avg_call_us": call_us}}
    if fact:
        res["config"] |= {"basis_rank": wl.basis_rank, "resid_rank_max": wl.resid_rank_max,
                          "rank16_frac": wl.rank16_frac}
        # the rate of an attention over rebuilt hd-wide rows doing the same job
        dense = prefill_flops(n, T, wl.n_q_heads, wl.head_dim)
        res["roofline"]["dense_equivalent_tflops"] = dense / (us * 1e-6) / 1e12
    res["roofline_alu"] = issue_roofline(wl, fact, us)
    calibration_copy()
    traffic = recorded_traffic(workload)
    if traffic is not None:
        res["roofline"]["traffic"] = traffic["bytes_per_launch"]
        res["roofline"]["traffic_source"] = traffic["source"]
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        hq = {l: qs[l].cpu() for l in layers}
        memo = {}
        if fact:
            def host_layer(l):
                if l not in memo:
                    memo.clear()
                    o = int(src[l, 0])
                    ck, cv = datagen.pair_coeffs(wl, o // 2, device="cuda")
                    bk, bv = datagen.pair_basis(wl, o // 2, device="cuda")
                    uk, uv = datagen.layer_residual_basis(wl, l, device="cuda")
                    dk, dv, sk, sv = datagen.layer_residual(wl, l, rank, device="cuda")
                    memo[l] = tuple(x.cpu() for x in (ck, cv, dk, dv, sk, sv, bk, bv, uk, uv, rank))
                return memo[l]
            res["cpu_baseline"] = cpu_fact_prefill(wl, layers, host_layer, hq, n)
        else:
            def host_kv(l):
                if l not in memo:
                    memo.clear()
                    k, v = datagen.owner_kv(wl, l, device="cuda")
                    memo[l] = (k.cpu(), v.cpu())
                return memo[l]
            res["cpu_baseline"] = cpu_prefill(wl, layers, host_kv, hq, n)
    print(json.dumps(res), flush=True)


def encode_call_bytes(wl, n, owner):
    """Algorithmic HBM bytes of one kvs_encode_factorized call over n tokens
    (batch 1): K and V rows of the layer in, and of the coefficient-writing
    layer when it is another one; the cache entries out (coefficients when
    the layer owns the pair's slot, ceil(r/8) code granules, a scale per
    token and KV head, the meta entry)."""
    H, hd = wl.n_kv_heads, wl.head_dim
    n_hi = int(round(wl.rank16_frac * n))
    granule_bytes = 8 * (2 * n_hi + (n - n_hi) // 2)          # ranks 16 / 8 / 0
    rows = 2 * n * H * hd * 2 * (1 if owner else 2)
    out = 2 * (H * (granule_bytes + 2 * n) + (n * H * wl.basis_rank * 2 if owner else 0)) + 2 * n
    return rows + out


def encode_main(args):
    """Factorized write path over a 4096-token prompt chunk on the 64K
    factorized model's shape (32 layers in 16 pairs, 32 q / 8 KV heads, hd
    128, basis rank 32, residual ranks 0/8/16 by seeded rank): a step encodes
    the chunk's K/V rows of every layer into the cache (kvs_encode_factorized;
    the pair's lower layer writes the coefficients, the upper one passes the
    lower layer's rows).  The bases of every pair and layer are built once
    from the same rows (kvs_pair_basis, kvs_residual_basis) and timed
    separately."""
    if args.gpus != 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        sys.exit(2)
    n = 4096
    wl = datagen.WORKLOADS["factorized_64k"].with_(batch=1, ctx=n)
    torch.cuda.set_device(0)
    log(f"[bench] setting up {ENCODE_WORKLOAD}: {n} tokens x {wl.n_layers} layers")
    src, w = datagen.share_map(wl)
    cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", 1, n,
                        kind=K.KVS_FACTORIZED, basis_rank=wl.basis_rank,
                        resid_rank_max=wl.resid_rank_max)
    plan = K.kvs_share_plan(cfg, src, w)
    cache = K.Cache(plan, "cuda")
    owners = datagen.owner_layers(src)
    rows = {}
    for pair in range(wl.n_layers // 2):
        ka, kb = datagen.correlated_pair_rows(wl, pair, "k", device="cuda")
        va, vb = datagen.correlated_pair_rows(wl, pair, "v", device="cuda")
        rows[2 * pair], rows[2 * pair + 1] = (ka, va), (kb, vb)
    rank = datagen.token_ranks(wl, device="cuda")
    start = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_tok = torch.full((1,), n, dtype=torch.int32, device="cuda")
    Hkv, R, Rm, hd = wl.n_kv_heads, wl.basis_rank, wl.resid_rank_max, wl.head_dim
    bk = cache.basis_k.view(torch.bfloat16).view(len(owners), Hkv, R, hd)
    bv = cache.basis_v.view(torch.bfloat16).view(len(owners), Hkv, R, hd)
    uk = cache.ubasis_k.view(torch.bfloat16).view(wl.n_layers, Hkv, Rm, hd)
    uv = cache.ubasis_v.view(torch.bfloat16).view(wl.n_layers, Hkv, Rm, hd)
    ews = torch.empty(K.kvs_encode_workspace_size(plan, 1, n), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # every pair's basis in one batched call, then every layer's residual
    # directions in one batched call, with a workspace that holds all items
    item = K.kvs_basis_workspace_size(plan, 1, n)
    bws = torch.empty(item * wl.n_layers, dtype=torch.uint8, device="cuda")

    def owner_of(l):
        return int(src[l, 0])

    def build_bases():
        K.kvs_pair_bases(plan, [rows[o][0] for o in owners], [rows[o][1] for o in owners],
                         [rows[o + 1][0] for o in owners], [rows[o + 1][1] for o in owners],
                         n_tok, [bk[i] for i in range(len(owners))],
                         [bv[i] for i in range(len(owners))], workspace=bws, stream=stream)
        L_all = list(range(wl.n_layers))
        slot = [owners.index(owner_of(l)) for l in L_all]
        K.kvs_residual_bases(plan, [rows[l][0] for l in L_all], [rows[l][1] for l in L_all],
                             [bk[slot[l]] for l in L_all], [bv[slot[l]] for l in L_all], n_tok,
                             [uk[l] for l in L_all], [uv[l] for l in L_all],
                             k_owner=[None if owner_of(l) == l else rows[owner_of(l)][0] for l in L_all],
                             v_owner=[None if owner_of(l) == l else rows[owner_of(l)][1] for l in L_all],
                             workspace=bws, stream=stream)

    build_bases()
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    build_bases()
    b1.record(stream)
    torch.cuda.synchronize()
    basis_ms = b0.elapsed_time(b1)

    ev = {l: [] for l in range(wl.n_layers)}

    def step(record=False):
        for l in range(wl.n_layers):
            k, v = rows[l]
            o = owner_of(l)
            ko, vo = (None, None) if o == l else rows[o]
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            K.kvs_encode_factorized(plan, cache, l, k, v, rank, start, k_owner=ko, v_owner=vo,
                                    workspace=ews, stream=stream)
            if record:
                e1.record(stream)
                ev[l].append((e0, e1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step(record=True)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    per = {l: sum(e0.elapsed_time(e1) for e0, e1 in ev[l]) * 1e3 / args.steps for l in ev}
    upper = [l for l in range(wl.n_layers) if owner_of(l) != l]
    us = sum(per[l] for l in upper) / len(upper)
    nbytes = encode_call_bytes(wl, n, owner=False)
    achieved = nbytes / (us * 1e-6) / 1e9
    res = {"metric": "factorized cache write path: encoded tokens/s (all layers) and HBM GB/s",
           "value": n * 1000.0 / ms, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": ENCODE_WORKLOAD, "layers": wl.n_layers, "batch": 1, "chunk": n,
                      "kv_heads": Hkv, "head_dim": hd, "basis_rank": R, "resid_rank_max": Rm,
                      "rank16_frac": wl.rank16_frac},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                        "kernel": "kvs_encode_factorized call of an upper pair layer "
                                  "(encode_kernel + fact_append_kernel)",
                        "bytes_per_launch": nbytes, "avg_launch_us": us,
                        "owner_layer_avg_us": sum(per[l] for l in owners) / len(owners)},
           "basis_build_ms": basis_ms,
           "basis_build": f"{len(owners)} pair bases + {wl.n_layers} residual bases "
                          f"(K and V) from {n} rows per layer, two batched calls"}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")

        def bases(l):
            s = owners.index(owner_of(l))
            return bk[s], bv[s], uk[l], uv[l]
        res["cpu_baseline"] = cpu_encode(wl, n, rows, owner_of, bases, rank)
    print(json.dumps(res), flush=True)



# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

class DecodeRig:
    """A workload's cache filled to its capacity (wl.batch sequences of
    wl.ctx tokens), its queries, and the new token each step appends at
    position ctx-1 of every sequence it runs.  Steps may run fewer sequences
    (the first B) and a shorter context (positions 0..ctx-1)."""

    def __init__(self, wl):
        self.wl = wl
        self.fact = wl.kind == "factorized"
        if self.fact:
            self.src, self.w, self.plan, self.cache, self.owners, self.rank = setup_factorized(wl)
        else:
            self.src, self.w, self.plan, self.cache, self.owners = setup(wl)
        L = wl.n_layers
        self.qs = [datagen.decode_q(wl, l, device="cuda") for l in range(L)]
        self.stream = torch.cuda.current_stream()
        if self.fact:
            one = wl.with_(ctx=1)
            r1 = self.rank[:, wl.ctx - 1:].contiguous()
            self.r1 = r1
            self.new_f = {}
            for l in range(L):
                cc = (datagen.pair_coeffs(one, 1000 + l, device="cuda") if l in self.owners
                      else (None, None))
                self.new_f[l] = cc + datagen.layer_residual(one, 1000 + l, r1, device="cuda")
        else:
            self.new_kv = {l: datagen.owner_kv(wl, 1000 + l, device="cuda", ctx=1) for l in self.owners}
        self.flush = torch.ones((FLUSH_BYTES // 4 // 4096, 4096), dtype=torch.float32, device="cuda")

    def call_bytes(self, l, B, ctx):
        wl = self.wl
        if self.fact:
            return fact_bytes_per_call(wl.with_(batch=B, ctx=ctx), self.rank[:B, :ctx])
        return bytes_per_call(wl.with_(batch=B, ctx=ctx), self.src, l)

    def point(self, B, ctx):
        """Callables and buffers of a step at batch B, context ctx."""
        wl, st = self.wl, self.stream
        L = wl.n_layers
        pos = torch.full((B,), ctx - 1, dtype=torch.int32, device="cuda")
        seq_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
        n_splits = K.kvs_decode_splits(self.plan, B, ctx)
        ws = torch.zeros(K.kvs_decode_workspace_size(self.plan, B, n_splits), dtype=torch.uint8,
                         device="cuda")
        outs = [torch.empty((B, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
                for _ in range(L)]
        qs = [q[:B].contiguous() for q in self.qs]
        if self.fact:
            r1 = self.rank[:B, ctx - 1:ctx].contiguous()
            new = {l: tuple(None if x is None else x[:B].contiguous() for x in v)
                   for l, v in self.new_f.items()}

            def append(l):
                ck, cv, dk, dv, sk, sv = new[l]
                K.kvs_append_factorized(self.plan, self.cache, l, ck, cv, dk, dv, sk, sv, r1, pos,
                                        stream=st)
        else:
            new = {l: (kv[0][:B].contiguous(), kv[1][:B].contiguous()) for l, kv in self.new_kv.items()}

            def append(l):
                if l in new:
                    K.kvs_append(self.plan, self.cache, l, new[l][0], new[l][1], pos, stream=st)

        def decode(l):
            K.kvs_attn_decode(self.plan, self.cache, l, qs[l], seq_len, ctx, out=outs[l],
                              n_splits=n_splits, workspace=ws, stream=st)

        return dict(append=append, decode=decode, n_splits=n_splits, qs=qs, seq_len=seq_len,
                    outs=outs, ws=ws)

    def warm_step_ms(self, pt, steps, warmup):
        L, st = self.wl.n_layers, self.stream

        def step():
            for l in range(L):
                pt["append"](l)
                pt["decode"](l)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(st)
        for _ in range(steps):
            step()
        t1.record(st)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def cold_step_ms(self, pt, passes):
        """A step with the cache flushed before each layer's calls: the sum of
        the per-layer intervals (append + decode), the flushes outside them."""
        L, st = self.wl.n_layers, self.stream
        ev = []
        for _ in range(passes):
            for l in range(L):
                self.flush.sum(dim=0)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                pt["append"](l)
                pt["decode"](l)
                e1.record(st)
                ev.append((e0, e1))
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / passes

    def launches(self, pt, layers, passes):
        """Cache-flushed decode launches of ``layers``: per-launch kernel time
        (events on the partition kernel) and call time (stream events)."""
        st = self.stream
        # warm both launch paths: the plain one and the timed one (its first
        # use sets up the extended launch)
        pt["decode"](layers[0])
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        K.kvs_time_next_launch(w0, w1, st)
        pt["decode"](layers[0])
        torch.cuda.synchronize()
        ev = []
        # one extra pass first, discarded: one-time costs of the first timed
        # launches (seen as a single call of tens of ms) stay out of the mean
        for i in range(passes + 1):
            for l in layers:
                self.flush.sum(dim=0)
                e0, e1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
                K.kvs_time_next_launch(k0, k1, st)
                e0.record(st)
                pt["decode"](l)
                e1.record(st)
                if i > 0:
                    ev.append((l, e0, e1, k0, k1))
        torch.cuda.synchronize()
        kern = [k0.elapsed_time(k1) * 1e3 for _, e0, e1, k0, k1 in ev]
        call = [e0.elapsed_time(e1) * 1e3 for _, e0, e1, k0, k1 in ev]
        return sum(kern) / len(kern), sum(call) / len(call), len(ev)

    def release(self):
        del self.cache, self.flush, self.qs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def decode_result(rig, args, cpu=True, step=True):
    """Warm and cold steps, the flushed per-launch roofline of the dominant
    kernel, and the oracle's CPU baseline for one decode workload."""
    wl = rig.wl
    L, B, ctx = wl.n_layers, wl.batch, wl.ctx
    src = rig.src
    pt = rig.point(B, ctx)
    res = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
           "data": "synthetic", "config": describe(wl, src) | {"n_splits": pt["n_splits"]}}
    step_bytes = sum(rig.call_bytes(l, B, ctx) for l in range(L))
    if step:
        ms = rig.warm_step_ms(pt, args.steps, args.warmup)
        ms_cold = rig.cold_step_ms(pt, passes=2)
        res |= {"value": B * 1000.0 / ms, "ms_per_step": ms,
                "step_hbm_gbs": step_bytes / (ms * 1e-3) / 1e9,
                "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "ms_per_step_cold": ms_cold,
                "value_cold": B * 1000.0 / ms_cold,
                "step_hbm_frac_cold": step_bytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "step_bytes": step_bytes}
    single = [l for l in range(L) if int(src[l, 1]) < 0]
    mixed = [l for l in range(L) if int(src[l, 1]) >= 0]
    dom = single if single else mixed
    us, call_us, n = rig.launches(pt, dom, args.roofline_passes)
    nbytes = rig.call_bytes(dom[0], B, ctx)
    achieved = nbytes / (us * 1e-6) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                       "kernel": ("fact_decode_kernel (factorized cache, split-K partitions)"
                                  if rig.fact else
                                  decode_kernel_name(wl, not single) + ", "
                                  + ("single-source layer" if single else "two-source layer")),
                       "bytes_per_launch": nbytes, "avg_launch_us": us,
                       "timing": "HIP events on the kernel's own start and end (hipExtLaunchKernel)",
                       "avg_call_us": call_us, "launches": n, "cache": "flushed"}
    if single and mixed:
        us2, call2, _ = rig.launches(pt, mixed, args.roofline_passes)
        b2 = rig.call_bytes(mixed[0], B, ctx)
        res["roofline_two_source"] = {"achieved": b2 / (us2 * 1e-6) / 1e9,
                                      "frac": b2 / (us2 * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                      "bytes_per_launch": b2, "avg_launch_us": us2,
                                      "avg_call_us": call2}
    ceil = read_ceiling(nbytes, rig.flush, rig.stream) if step else None
    if ceil is not None:
        res["roofline"]["read_ceiling"] = ceil
        res["roofline"]["frac_of_read_ceiling"] = achieved / ceil["gbs"]
    if step and "roofline_two_source" in res:
        c2 = read_ceiling(res["roofline_two_source"]["bytes_per_launch"], rig.flush, rig.stream)
        if c2 is not None:
            res["roofline_two_source"]["read_ceiling_gbs"] = c2["gbs"]
            res["roofline_two_source"]["frac_of_read_ceiling"] = (
                res["roofline_two_source"]["achieved"] / c2["gbs"])
    if rig.fact and step:
        res["router"] = router_result(rig, pt, dom, args, us, call_us)
    traffic = recorded_traffic(wl.name)
    if traffic is not None:
        res["roofline"]["traffic"] = traffic["bytes_per_launch"]
        res["roofline"]["traffic_source"] = traffic["source"]
    if cpu:
        log(f"[bench] cpu baseline: {wl.name}")
        res["cpu_baseline"] = cpu_fact_decode(rig) if rig.fact else cpu_dense_decode(rig)
    return res


READ_LAUNCH_SHAPES = [(blocks, u) for blocks in (256, 512, 1024, 2048, 4096) for u in (4, 8, 16)]


def read_ceiling(nbytes, flush, stream, reps=5):
    """What a plain read of the same bytes achieves on this GPU: the kernel of
    bench_read.hip (block-contiguous 16-byte non-temporal loads, nothing
    computed) over a buffer of ``nbytes``, cache flushed before each launch,
    timed with events on the kernel itself, as the decode kernels are; the
    median of ``reps`` launches for each of
    READ_LAUNCH_SHAPES, the fastest shape reported.  None if the probe
    library is not built."""
    import ctypes
    path = os.path.join(ROOT, "bench_read.so")
    if not os.path.exists(path):
        log("[bench] bench_read.so not built: no read ceiling")
        return None
    lib = ctypes.CDLL(path)
    lib.stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    n = (int(nbytes) + 15) // 16 * 16
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4096 * 256, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    best = None
    for blocks, u in READ_LAUNCH_SHAPES:
        if lib.stream_read(buf.data_ptr(), n, sink.data_ptr(), blocks, u, sp, None, None) != 0:
            raise RuntimeError("stream_read launch failed")
        ev = []
        for _ in range(reps):
            flush.sum(dim=0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)      # creates the events; the launch records them again
            e1.record(stream)
            if lib.stream_read(buf.data_ptr(), n, sink.data_ptr(), blocks, u, sp,
                               ctypes.c_void_p(e0.cuda_event), ctypes.c_void_p(e1.cuda_event)) != 0:
                raise RuntimeError("stream_read launch failed")
            ev.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)[reps // 2]
        if best is None or t < best[0]:
            best = (t, blocks, u)
    del buf, sink
    t, blocks, u = best
    return {"bytes": n, "us": t, "gbs": n / (t * 1e-6) / 1e9, "frac_of_peak": n / (t * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "launch": f"{blocks} workgroups x 256 threads, {u} loads in flight per thread",
            "timing": "HIP events on the kernel's own start and end (median of %d launches, fastest of %d "
                      "launch shapes), cache flushed" % (reps, len(READ_LAUNCH_SHAPES))}


def router_result(rig, pt, dom, args, us, call_us):
    """Router statistics: the same cache-flushed launches with the entropy and
    peak side output, then the rank choice over every layer's statistics."""
    wl, st = rig.wl, rig.stream
    L, B = wl.n_layers, wl.batch
    stats = torch.empty((L, B, wl.n_q_heads, 2), dtype=torch.float32, device="cuda")
    ev_s = []
    for _ in range(args.roofline_passes):
        for l in dom:
            rig.flush.sum(dim=0)
            e0, e1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            K.kvs_time_next_launch(k0, k1, st)
            e0.record(st)
            K.kvs_attn_decode_stats(rig.plan, rig.cache, l, pt["qs"][l], pt["seq_len"], wl.ctx,
                                    out=pt["outs"][l], stats=stats[l], n_splits=pt["n_splits"],
                                    workspace=pt["ws"], stream=st)
            e1.record(st)
            ev_s.append((e0, e1, k0, k1))
    router = K.kvs_router(0.5, 0.8, 0.5, wl.resid_rank_max, wl.resid_rank_max // 2, 0)
    ranks = torch.empty(B, dtype=torch.uint8, device="cuda")
    K.kvs_route_ranks(rig.plan, stats, pt["seq_len"], router, rank_out=ranks, stream=st)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(st)
    for _ in range(10):
        K.kvs_route_ranks(rig.plan, stats, pt["seq_len"], router, rank_out=ranks, stream=st)
    r1.record(st)
    torch.cuda.synchronize()
    us_s = sum(k0.elapsed_time(k1) for e0, e1, k0, k1 in ev_s) * 1e3 / len(ev_s)
    call_s = sum(e0.elapsed_time(e1) for e0, e1, k0, k1 in ev_s) * 1e3 / len(ev_s)
    return {"decode_with_stats_us": us_s, "decode_us": us, "stats_overhead_frac": us_s / us - 1.0,
            "call_with_stats_us": call_s, "call_us": call_us,
            "stats_overhead_call_frac": call_s / call_us - 1.0,
            "route_us": r0.elapsed_time(r1) * 1e3 / 10, "route_sets": L,
            "routed_ranks": ranks.cpu().tolist()}


def decode_main(args):
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is a "
              "single-GPU kernel library; sharding across GPUs is described, not built.",
              file=sys.stderr)
        sys.exit(2)
    wl = datagen.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    log(f"[bench] setting up {wl.name}")
    rig = DecodeRig(wl)
    if args.roofline_only:
        res = decode_result(rig, args, cpu=False, step=False)
        rig.release()
        calibration_copy()
        print(json.dumps(res), flush=True)
        return
    res = decode_result(rig, args, cpu=not args.no_cpu_baseline)
    rig.release()
    del rig
    if args.workload == DEFAULT_WORKLOAD and not args.no_extras:
        # the 64K factorized decode beside the dense one
        log("[bench] setting up factorized_64k")
        frig = DecodeRig(datagen.WORKLOADS["factorized_64k"])
        f = decode_result(frig, args, cpu=not args.no_cpu_baseline)
        frig.release()
        del frig
        res["roofline_factorized"] = f["roofline"] | {
            "workload": "factorized_64k", "config": f["config"], "value": f["value"],
            "value_unit": "tokens/s", "ms_per_step": f["ms_per_step"],
            "ms_per_step_cold": f["ms_per_step_cold"], "step_hbm_frac": f["step_hbm_frac"],
            "router": f["router"]} | ({"cpu_baseline": f["cpu_baseline"]} if "cpu_baseline" in f else {})
        # the 4-layer fp32 toy step (parity-sized; latency only)
        trig = DecodeRig(datagen.WORKLOADS["tiny_cla2"])
        tpt = trig.point(1, trig.wl.ctx)
        res["tiny_cla2"] = {"us_per_step": trig.warm_step_ms(tpt, 50, 10) * 1e3,
                            "layers": trig.wl.n_layers, "batch": 1, "ctx": trig.wl.ctx,
                            "dtype": "f32", "what": "append + decode of every layer, warm"}
        trig.release()
    calibration_copy()
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------
# the batch x context grid
# ----------------------------------------------------------------------------

SWEEP = (("tinyllama_cla2", (1, 8, 16, 32, 64, 128), (512, 1024, 2048)),
         ("cla2_64k", (1, 2, 4, 8), (16384, 32768, 65536)))


SWEEP_HEADER = """# Decode throughput per batch x context (one MI355X)

Command (repository root):

```
python3 bench.py --sweep --steps 10 --warmup 3 --sweep-out profiles/decode_sweep_batch_ctx.md
```

Each row: one decode step over all layers (append + decode per layer), one token per sequence. *warm*: back-to-back steps. *cold*: the 256 MB Infinity Cache flushed before every layer's calls (flush outside the timed intervals). *kernel*: the single-source decode kernel alone, HIP events on its own start and end, cache flushed before each launch. Rates are algorithmic bytes (every source K/V tile read once) per second; % of the 8 TB/s HBM peak. *plain read*: `bench_read.hip` reading a buffer of the call's byte count once (block-contiguous 16-byte non-temporal loads, nothing computed), the same kernel events and cache flush, the fastest of 15 launch shapes (median of 3 launches each): what one launch that reads those bytes reaches on this GPU. `tinyllama_cla2`: 22 layers (11 owners), 32 q / 4 KV heads, hd 64. `cla2_64k`: 32 layers (16 owners), 32 q / 8 KV heads, hd 128, 1% of keys x4. Splits: the library's split-K partition count for the point.

"""


def sweep_main(args):
    if args.gpus != 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    points = []
    for name, batches, ctxs in SWEEP:
        base = datagen.WORKLOADS[name]
        wl = base.with_(batch=max(batches), ctx=max(ctxs))
        log(f"[sweep] setting up {name} at capacity B={wl.batch} ctx={wl.ctx}")
        rig = DecodeRig(wl)
        single = [l for l in range(wl.n_layers) if int(rig.src[l, 1]) < 0]
        for ctx in ctxs:
            for B in batches:
                pt = rig.point(B, ctx)
                ms = rig.warm_step_ms(pt, args.steps, args.warmup)
                ms_cold = rig.cold_step_ms(pt, passes=1)
                us, call_us, _ = rig.launches(pt, single, 1)
                step_bytes = sum(rig.call_bytes(l, B, ctx) for l in range(wl.n_layers))
                nbytes = rig.call_bytes(single[0], B, ctx)
                p = {"workload": name, "batch": B, "ctx": ctx, "n_splits": pt["n_splits"],
                     "tokens_s": B * 1000.0 / ms, "ms_per_step": ms,
                     "step_gbs": step_bytes / (ms * 1e-3) / 1e9,
                     "tokens_s_cold": B * 1000.0 / ms_cold, "ms_per_step_cold": ms_cold,
                     "step_gbs_cold": step_bytes / (ms_cold * 1e-3) / 1e9,
                     "kernel_us": us, "kernel_gbs": nbytes / (us * 1e-6) / 1e9,
                     "call_us": call_us, "bytes_per_call": nbytes}
                for k in ("step_gbs", "step_gbs_cold", "kernel_gbs"):
                    p[k.replace("gbs", "frac")] = p[k] / HBM_PEAK_GBS
                ceil = read_ceiling(nbytes, rig.flush, rig.stream, reps=3)
                if ceil is not None:
                    p["read_ceiling_gbs"] = ceil["gbs"]
                    p["kernel_frac_of_read"] = p["kernel_gbs"] / ceil["gbs"]
                points.append(p)
                log(f"[sweep] {name} B={B} ctx={ctx}: {p['tokens_s']:.0f} tok/s, kernel "
                    f"{p['kernel_frac']:.1%} of HBM peak, cold step {p['step_frac_cold']:.1%}")
                del pt
        rig.release()
        del rig
    if args.sweep_out:
        lines = ["| workload | batch | ctx | splits | tok/s (warm) | step GB/s (% peak) | "
                 "tok/s (cold) | cold step GB/s (% peak) | kernel us | kernel GB/s (% peak) | "
                 "plain read of the call's bytes, GB/s | kernel / plain read |",
                 "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for p in points:
            rd = (f"{p['read_ceiling_gbs']:,.0f} | {p['kernel_frac_of_read']:.1%}"
                  if "read_ceiling_gbs" in p else "- | -")
            lines.append(f"| {p['workload']} | {p['batch']} | {p['ctx']} | {p['n_splits']} | "
                         f"{p['tokens_s']:,.0f} | {p['step_gbs']:,.0f} ({p['step_frac']:.1%}) | "
                         f"{p['tokens_s_cold']:,.0f} | {p['step_gbs_cold']:,.0f} "
                         f"({p['step_frac_cold']:.1%}) | {p['kernel_us']:.1f} | "
                         f"{p['kernel_gbs']:,.0f} ({p['kernel_frac']:.1%}) | {rd} |")
        open(args.sweep_out, "w").write(SWEEP_HEADER + "\n".join(lines) + "\n")
    print(json.dumps({"metric": METRIC, "sweep": points}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=["tiny_cla2", "tinyllama_cla2", "depthgraft", "cla2_64k",
                             "factorized_64k", "tinyllama_cla2_top", *PREFILL_WORKLOADS,
                             ENCODE_WORKLOAD])
    ap.add_argument("--roofline-passes", type=int, default=3)
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the cache-flushed per-launch timing loop (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload only: skip the factorized and toy extras")
    ap.add_argument("--sweep", action="store_true", help="time the batch x context grid")
    ap.add_argument("--sweep-out", metavar="FILE", help="with --sweep: markdown table to FILE")
    ap.add_argument("--summarize", metavar="PROFILE_DIR",
                    help="print the counter summary of a rocprofv3 profile directory and exit")
    ap.add_argument("--kernel", default="decode_kernel",
                    help="kernel name, or one instantiation such as "
                         "'decode_kernel<unsigned short, 128, 4, 1>'")
    ap.add_argument("--record", action="store_true",
                    help="with --summarize: write profiles/<kernel>_<workload>.md and "
                         "the workload's entry of profiles/traffic.json")
    ap.add_argument("--prefill", action="store_true",
                    help="time the DepthGraft causal prefill chunk instead of decode")
    args = ap.parse_args()
    if args.summarize:
        s = summarize(args.summarize, args.kernel, args.workload)
        s["source_sha256_16"] = source_digest(args.kernel)
        print(json.dumps(s, indent=1))
        if args.record:
            print(record_profile(args.summarize, args.kernel, args.workload, s))
        return
    # Cyclic garbage collection off for the timed work: a collection pass
    # that lands between a call's two stream events (tens of ms with this
    # many live objects) leaves the GPU idle inside the interval and shows
    # up as one call of that length.  Reference counting still frees.
    gc.collect()
    gc.disable()
    if args.sweep:
        return sweep_main(args)
    if args.workload == ENCODE_WORKLOAD:
        return encode_main(args)
    if args.workload in PREFILL_WORKLOADS:
        return prefill_main(args, args.workload)
    if args.prefill:
        return prefill_main(args, PREFILL_WORKLOAD)
    return decode_main(args)


if __name__ == "__main__":
    main()
