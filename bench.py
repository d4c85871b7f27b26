"""Shared-KV decode attention benchmark on one MI355X.

A step is one decode step of the whole hot path over all layers of the
workload: every owner layer appends its new token's K/V (kvs_append, n=1),
then every layer runs split-K decode attention over its source slot(s)
(kvs_attn_decode: the partition kernel, plus a small merge kernel when the
sequence is split into several partitions).  The factorized workload
appends the new token's coefficients, codes, scales and rank
(kvs_append_factorized) instead of K/V.  Inputs are
resident in HBM before the timed region; K/V and queries are seeded
synthetic N(0,1) tensors of the workload's shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--roofline-only] [--no-cpu-baseline]

Prints one JSON line.  ``value`` is decode tokens/s (one token per sequence
per step, warm back-to-back steps).  ``roofline`` rates the decode launch of
a single-source layer against the 8 TB/s HBM peak with its algorithmic bytes
(every source tile, K and V, read once): its duration is timed with a pair
of HIP events that the library attaches to the decode kernel's own start and
end (kvs_time_next_launch, i.e. hipExtLaunchKernel; the partition merge and
the launch latency are reported apart as avg_call_us), with the 256 MB
Infinity Cache flushed before each launch by reading a 512 MB buffer (a read
leaves no dirty lines whose write-back would compete with the timed launch),
so no byte of the timed launch is served from a cache.
``cpu_baseline`` times the fp64 oracle on a bounded sample of sequences.
"""
import argparse
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


def cpu_baseline(wl, src, w, host_seq, budget_s=12.0):
    """fp64 oracle, single-threaded BLAS, over whole decode steps (all layers)
    of one sequence after another (cycling through the batch) until about
    ``budget_s`` of CPU time."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    done = 0
    elapsed = 0.0
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            kk, vv, qs = host_seq(done % wl.batch)
            t0 = time.perf_counter()
            for l in range(wl.n_layers):
                A.layer_decode(src.tolist(), w.tolist(), l, kk, vv, qs[l], [wl.ctx])
            elapsed += time.perf_counter() - t0
            done += 1
    return {"value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequence decode steps (cycling through the {wl.batch} sequences), "
                      f"each over all {wl.n_layers} layers at ctx {wl.ctx}, {elapsed:.1f} s "
                      f"(bf16->fp64 upcast included)"}


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
    cmd = (f"python3 bench.py --workload {workload} --steps 8 --warmup 2" if prefill
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
    if wl.dtype == "bf16" and wl.head_dim == 64 and not two_source and G <= 16:
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
        kernel = "fact_prefill_kernel (bf16 MFMA in the coefficient space, causal)"
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
    calibration_copy()
    traffic = recorded_traffic(workload)
    if traffic is not None:
        res["roofline"]["traffic"] = traffic["bytes_per_launch"]
        res["roofline"]["traffic_source"] = traffic["source"]
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
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tinyllama_cla2",
                    choices=["tiny_cla2", "tinyllama_cla2", "depthgraft", "cla2_64k",
                             "factorized_64k", "tinyllama_cla2_top", *PREFILL_WORKLOADS,
                             ENCODE_WORKLOAD])
    ap.add_argument("--roofline-passes", type=int, default=3)
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the cache-flushed per-launch timing loop (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    if args.workload == ENCODE_WORKLOAD:
        return encode_main(args)
    if args.workload in PREFILL_WORKLOADS:
        return prefill_main(args, args.workload)
    if args.prefill:
        return prefill_main(args, PREFILL_WORKLOAD)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is a "
              "single-GPU kernel library; sharding across GPUs is described, not built.",
              file=sys.stderr)
        sys.exit(2)

    wl = datagen.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    log(f"[bench] setting up {wl.name}")
    fact = wl.kind == "factorized"
    if fact:
        src, w, plan, cache, owners, rank = setup_factorized(wl)
    else:
        src, w, plan, cache, owners = setup(wl)
    L, B = wl.n_layers, wl.batch
    qs = [datagen.decode_q(wl, l, device="cuda") for l in range(L)]
    # the step's token lands at position ctx-1 (rewritten every step); the
    # query attends over ctx keys including it
    pos = torch.full((B,), wl.ctx - 1, dtype=torch.int32, device="cuda")
    if fact:
        one = wl.with_(ctx=1)
        r1 = rank[:, wl.ctx - 1:].contiguous()
        new_f = {}
        for l in range(L):
            cc = datagen.pair_coeffs(one, 1000 + l, device="cuda") if l in owners else (None, None)
            new_f[l] = cc + datagen.layer_residual(one, 1000 + l, r1, device="cuda")

        def append(l):
            ck, cv, dk, dv, sk, sv = new_f[l]
            K.kvs_append_factorized(plan, cache, l, ck, cv, dk, dv, sk, sv, r1, pos,
                                    stream=stream)
        call_bytes = [fact_bytes_per_call(wl, rank)] * L
    else:
        new_kv = {l: datagen.owner_kv(wl, 1000 + l, device="cuda", ctx=1) for l in owners}

        def append(l):
            if l in new_kv:
                K.kvs_append(plan, cache, l, new_kv[l][0], new_kv[l][1], pos, stream=stream)
        call_bytes = [bytes_per_call(wl, src, l) for l in range(L)]
    seq_len = torch.full((B,), wl.ctx, dtype=torch.int32, device="cuda")
    n_splits = K.kvs_decode_splits(plan, B, wl.ctx)
    ws = torch.zeros(K.kvs_decode_workspace_size(plan, B, n_splits), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty((B, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(L)]
    stream = torch.cuda.current_stream()

    def decode(l):
        K.kvs_attn_decode(plan, cache, l, qs[l], seq_len, wl.ctx, out=outs[l],
                          n_splits=n_splits, workspace=ws, stream=stream)

    def step():
        for l in range(L):
            append(l)
            decode(l)

    res = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
           "data": "synthetic", "config": describe(wl, src) | {"n_splits": n_splits}}

    if not args.roofline_only:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        step_bytes = sum(call_bytes)
        res |= {"value": B * 1000.0 / ms, "ms_per_step": ms,
                "step_hbm_gbs": step_bytes / (ms * 1e-3) / 1e9,
                "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    # ---- per-launch roofline: cache flushed before every launch
    flush = torch.ones((FLUSH_BYTES // 4 // 4096, 4096), dtype=torch.float32, device="cuda")
    single = [l for l in range(L) if int(src[l, 1]) < 0]
    mixed = [l for l in range(L) if int(src[l, 1]) >= 0]
    timed = {}
    for group in (single, mixed):
        for l in group[:1]:
            decode(l)                                     # warm the launch path
        for _ in range(args.roofline_passes):
            for l in group:
                flush.sum(dim=0)
                e0, e1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
                K.kvs_time_next_launch(k0, k1, stream)
                e0.record(stream)
                decode(l)
                e1.record(stream)
                timed.setdefault(l, []).append((e0, e1, k0, k1))
    torch.cuda.synchronize()

    def avg_us(layers, kernel_only=True):
        d = [(k0.elapsed_time(k1) if kernel_only else e0.elapsed_time(e1)) * 1e3
             for l in layers for (e0, e1, k0, k1) in timed[l]]
        return sum(d) / len(d)

    dom = single if single else mixed
    us = avg_us(dom)
    nbytes = call_bytes[dom[0]]
    achieved = nbytes / (us * 1e-6) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                       "kernel": ("fact_decode_kernel (factorized cache, split-K partitions)"
                                  if fact else
                                  decode_kernel_name(wl, not single) + ", "
                                  + ("single-source layer" if single else "two-source layer")),
                       "bytes_per_launch": nbytes, "avg_launch_us": us,
                       "timing": "HIP events on the kernel's own start and end (hipExtLaunchKernel)",
                       "avg_call_us": avg_us(dom, kernel_only=False),
                       "launches": sum(len(timed[l]) for l in dom), "cache": "flushed"}
    if single and mixed:
        us2 = avg_us(mixed)
        b2 = call_bytes[mixed[0]]
        res["roofline_two_source"] = {"achieved": b2 / (us2 * 1e-6) / 1e9,
                                      "frac": b2 / (us2 * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                      "bytes_per_launch": b2, "avg_launch_us": us2,
                                      "avg_call_us": avg_us(mixed, kernel_only=False)}
    if fact:
        # router statistics: the same cache-flushed launches with the entropy
        # and peak side output, then the rank choice over every layer's
        # statistics
        stats = torch.empty((L, B, wl.n_q_heads, 2), dtype=torch.float32, device="cuda")
        ev_s = []
        for _ in range(args.roofline_passes):
            for l in dom:
                flush.sum(dim=0)
                e0, e1, k0, k1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
                K.kvs_time_next_launch(k0, k1, stream)
                e0.record(stream)
                K.kvs_attn_decode_stats(plan, cache, l, qs[l], seq_len, wl.ctx, out=outs[l],
                                        stats=stats[l], n_splits=n_splits, workspace=ws,
                                        stream=stream)
                e1.record(stream)
                ev_s.append((e0, e1, k0, k1))
        router = K.kvs_router(0.5, 0.8, 0.5, wl.resid_rank_max, wl.resid_rank_max // 2, 0)
        ranks = torch.empty(B, dtype=torch.uint8, device="cuda")
        K.kvs_route_ranks(plan, stats, seq_len, router, rank_out=ranks, stream=stream)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for _ in range(10):
            K.kvs_route_ranks(plan, stats, seq_len, router, rank_out=ranks, stream=stream)
        r1.record(stream)
        torch.cuda.synchronize()
        us_s = sum(k0.elapsed_time(k1) for e0, e1, k0, k1 in ev_s) * 1e3 / len(ev_s)
        call_s = sum(e0.elapsed_time(e1) for e0, e1, k0, k1 in ev_s) * 1e3 / len(ev_s)
        call = res["roofline"]["avg_call_us"]
        res["router"] = {"decode_with_stats_us": us_s, "decode_us": us,
                         "stats_overhead_frac": us_s / us - 1.0,
                         "call_with_stats_us": call_s, "call_us": call,
                         "stats_overhead_call_frac": call_s / call - 1.0,
                         "route_us": r0.elapsed_time(r1) * 1e3 / 10,
                         "route_sets": L, "routed_ranks": ranks.cpu().tolist()}
    del flush
    calibration_copy()
    traffic = recorded_traffic(wl.name)
    if traffic is not None:
        res["roofline"]["traffic"] = traffic["bytes_per_launch"]
        res["roofline"]["traffic_source"] = traffic["source"]

    if not args.roofline_only and not args.no_cpu_baseline and not fact:
        log("[bench] cpu baseline")
        full = {}
        for l in owners:
            k, v = datagen.owner_kv(wl, l, device="cuda")
            k[:, wl.ctx - 1:] = new_kv[l][0]
            v[:, wl.ctx - 1:] = new_kv[l][1]
            full[l] = (k, v)

        def host_seq(b):
            kk = {l: full[l][0][b:b + 1].cpu() for l in owners}
            vv = {l: full[l][1][b:b + 1].cpu() for l in owners}
            return kk, vv, [q[b:b + 1].cpu() for q in qs]

        res["cpu_baseline"] = cpu_baseline(wl, src, w, host_seq)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
