"""GPU parity of top/middle configurations (a source above its reader) with
diagonal masking, against the oracle: such a layer's decode query skips the
current position and its causal prefill query at position P sees keys
0..P-1 ("A Systematic Study of Cross-Layer KV Sharing for Efficient LLM
Inference", TL;DR: top/middle configurations, diagonal masking)."""
import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from oracle import plan as P
from tests._gpu_harness import Dense, Factorized, assert_close, note

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS

DECODE = {
    # name: (workload, batch, ctx, lens)
    "top_cla2_hd64_g8": (W["tinyllama_cla2"].with_(n_layers=4, share="cla2_top"), 3, 300, [300, 1, 65]),
    "mid3_hd128_g4": (W["cla2_64k"].with_(n_layers=6, share="mid3"), 2, 700, [700, 129]),
    "top_tiny_f32": (W["tiny_cla2"].with_(share="cla2_top"), 2, 128, [128, 2]),
}


@pytest.mark.parametrize("case", list(DECODE))
def test_top_middle_decode_matches_oracle(case):
    wl, B, ctx, lens = DECODE[case]
    note(f"[top/middle decode] {case}: lens={lens}")
    d = Dense(wl, B, ctx, lens)
    src, w = d.src.tolist(), d.w.tolist()
    assert any(P.excludes_current(src, w, l) for l in range(wl.n_layers))
    for l in range(wl.n_layers):
        li = K.kvs_plan_layer(d.plan, l)
        assert li.masks_current == int(P.excludes_current(src, w, l))
        got = d.decode(l)
        torch.cuda.synchronize()
        assert_close(got, d.oracle_decode(l), wl.dtype, f"{case} layer {l}")


def test_masked_layer_with_one_token_is_zero():
    """seq_len 1: the masked layer has no key at all (zeros); its source layer
    sees its own entry."""
    wl = W["tinyllama_cla2"].with_(n_layers=2, share="cla2_top")
    d = Dense(wl, 2, 64, [1, 1])
    got = d.decode(0)
    torch.cuda.synchronize()
    assert float(got.abs().max()) == 0.0
    assert_close(d.decode(1), d.oracle_decode(1), "bf16", "source layer")


PREFILL = {
    # name: (workload, batch, ctx, lens, n)
    "top_hd128_offset0": (W["cla2_64k"].with_(n_layers=2, share="cla2_top"), 1, 256, [256], 256),
    "top_hd128_ragged": (W["cla2_64k"].with_(n_layers=2, share="cla2_top"), 2, 320, [300, 190], 130),
    "mid3_hd64_g8": (W["tinyllama_cla2"].with_(n_layers=3, share="mid3"), 2, 200, [200, 97], 97),
}


@pytest.mark.parametrize("case", list(PREFILL))
def test_top_middle_prefill_matches_oracle(case):
    wl, B, ctx, lens, n = PREFILL[case]
    note(f"[top/middle prefill] {case}: lens={lens} n={n}")
    d = Dense(wl, B, ctx, lens)
    for l in range(wl.n_layers):
        q = datagen.prefill_q(wl, l, n, batch=B)
        got = K.kvs_attn_prefill_chunk(d.plan, d.cache, l, q.cuda(), d.seq_len, causal=True)
        torch.cuda.synchronize()
        ref = A.layer_prefill(d.src.tolist(), d.w.tolist(), l, d.k, d.v, q, lens, causal=True)
        assert_close(got, ref, "bf16", f"{case} layer {l}")
        if P.excludes_current(d.src.tolist(), d.w.tolist(), l) and lens[0] == n:
            assert float(got[0, 0].abs().max()) == 0.0     # position 0 sees no key


def test_top_factorized_decode_matches_oracle():
    wl = W["factorized_64k"].with_(n_layers=4, n_q_heads=8, n_kv_heads=2, share="pairs_top")
    d = Factorized(wl, 2, 300, [300, 150])
    for l in range(wl.n_layers):
        got = d.decode(l)
        torch.cuda.synchronize()
        assert_close(got, d.oracle_decode(l), "bf16", f"factorized top layer {l}")
