"""Randomized parity sweep: seeded random shapes (head dim, dtype, KV heads,
group size, sharing map, batch, ragged lengths, split count) through the
C ABI against the fp64 oracle, decode and prefill, dense and factorized.
The cases are drawn once from a fixed seed, so the sweep is the same on
every run; shapes the library does not implement are not drawn."""
import random

import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from tests._gpu_harness import Dense, Factorized, assert_close, note

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS


def _draw(n_cases=48, seed=20261203):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n_cases:
        kind = rng.choice(["dense", "dense", "dense", "fact"])
        hd = rng.choice([64, 128])
        hkv = rng.choice([1, 2, 4, 8])
        B = rng.randint(1, 3)
        if kind == "dense":
            dtype = rng.choice(["bf16", "bf16", "bf16", "f32"])
            gs = [1, 2, 4, 8, 16] + ([32] if hd == 64 else [])
            g = rng.choice(gs if dtype == "bf16" else [1, 2, 4, 8])
            share = rng.choice(["cla2", "cla2_top", "mid3", "identity", "depthgraft"])
            if share == "depthgraft" and g > 8:        # no two-source kernel for G > 8
                continue
            ctx = rng.choice([64, 100, 257, 640, 1300])
        else:
            dtype, g = "bf16", rng.choice([1, 2, 4, 8])
            share = rng.choice(["pairs", "pairs_top"])
            ctx = rng.choice([64, 130, 500, 1100])
        lens = [rng.choice([0, 1, rng.randint(1, ctx), ctx]) for _ in range(B)]
        if max(lens) == 0:
            lens[0] = ctx
        cases.append(dict(kind=kind, hd=hd, hkv=hkv, g=g, dtype=dtype, share=share, B=B, ctx=ctx,
                          lens=lens, splits=rng.choice([0, 0, 1, 3, 17]), causal=rng.random() < 0.8,
                          r16=rng.choice([0.0, 0.1, 0.5, 1.0]), pick=rng.random()))
    return cases


CASES = _draw()


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape_matches_oracle(i):
    c = CASES[i]
    note(f"[sweep {i}] {c}")
    rng = random.Random(c["pick"])
    if c["kind"] == "dense":
        base = W["cla2_64k"] if c["hd"] == 128 else W["tinyllama_cla2"]
        L = 6 if c["share"] == "depthgraft" else 4
        kw = dict(n_layers=L, n_q_heads=c["hkv"] * c["g"], n_kv_heads=c["hkv"], head_dim=c["hd"],
                  dtype=c["dtype"], share=c["share"])
        if c["share"] == "depthgraft":
            kw["dg_stride"] = 2
        wl = base.with_(**kw)
        d = Dense(wl, c["B"], c["ctx"], c["lens"])
        layers = rng.sample(range(L), 3)
        for l in layers:
            got = d.decode(l, n_splits=c["splits"])
            torch.cuda.synchronize()
            assert_close(got, d.oracle_decode(l), c["dtype"], f"decode layer {l}")
        if c["dtype"] == "bf16":
            l = layers[0]
            n = rng.randint(1, min(x for x in c["lens"] if x > 0))
            q = datagen.prefill_q(wl, l, n, batch=c["B"])
            got = K.kvs_attn_prefill_chunk(d.plan, d.cache, l, q.cuda(), d.seq_len, causal=c["causal"])
            torch.cuda.synchronize()
            ref = A.layer_prefill(d.src.tolist(), d.w.tolist(), l, d.k, d.v, q, c["lens"], causal=c["causal"])
            assert_close(got, ref, "bf16", f"prefill layer {l} n {n}")
    else:
        wl = W["factorized_64k"].with_(n_layers=4, n_q_heads=c["hkv"] * c["g"], n_kv_heads=c["hkv"],
                                       head_dim=c["hd"], share=c["share"], rank16_frac=c["r16"])
        f = Factorized(wl, c["B"], c["ctx"], c["lens"])
        layers = rng.sample(range(4), 2)
        for l in layers:
            got = f.decode(l, n_splits=c["splits"])
            torch.cuda.synchronize()
            assert_close(got, f.oracle_decode(l), "bf16", f"factorized decode layer {l}")
        l = layers[0]
        n = rng.randint(1, min(x for x in c["lens"] if x > 0))
        q = datagen.prefill_q(wl, l, n, batch=c["B"])
        assert_close(f.prefill(l, q, causal=c["causal"]), f.oracle_prefill(l, q, causal=c["causal"]), "bf16",
                     f"factorized prefill layer {l} n {n}")
