"""GPU parity of the factorized-cache prefill chunk (scores and values
contracted in the 48-wide coefficient space on MFMA) against the oracle's
explicit per-token reconstruction followed by plain causal attention."""
import numpy as np
import pytest
import torch

import datagen
from oracle import attention as A
from tests._gpu_harness import Factorized, assert_close, errors, note, TOL_ABS

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
F = W["factorized_64k"]

CASES = {
    # name: (workload, batch, ctx, lens, n, causal)
    "g4_hd128_ragged": (F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2), 2, 300, [300, 150], 130, True),
    "g4_hd128_offset0": (F.with_(n_layers=2), 1, 256, [256], 256, True),
    "g4_hd128_noncausal": (F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2), 2, 200, [200, 77], 64, False),
    "g8_hd64": (F.with_(n_layers=2, n_q_heads=16, n_kv_heads=2, head_dim=64), 2, 260, [260, 100], 100, True),
    "g1_hd64": (F.with_(n_layers=2, n_q_heads=2, n_kv_heads=2, head_dim=64), 2, 129, [129, 33], 33, True),
    "g2_hd128_top": (F.with_(n_layers=4, n_q_heads=4, n_kv_heads=2, share="pairs_top"), 2, 190,
                     [190, 70], 70, True),
    # few keys per early row, so single keys dominate rows: the absorbed
    # queries must not be rounded to bf16 alone
    "g8_hd128_few_keys": (F.with_(n_layers=4, n_q_heads=64, n_kv_heads=8), 1, 500, [57], 50, True),
    "g8_hd128_few_keys_full": (F.with_(n_layers=4, n_q_heads=64, n_kv_heads=8), 1, 500, [57], 50, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_factorized_prefill_matches_oracle(case):
    wl, B, ctx, lens, n, causal = CASES[case]
    note(f"[factorized prefill parity] {case}: L={wl.n_layers} B={B} lens={lens} n={n} "
         f"causal={causal} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} hd={wl.head_dim} share={wl.share}")
    d = Factorized(wl, B, ctx, lens)
    for l in range(wl.n_layers):
        q = datagen.prefill_q(wl, l, n, batch=B)
        got = d.prefill(l, q, causal=causal)
        assert_close(got, d.oracle_prefill(l, q, causal=causal), "bf16", f"{case} layer {l}")


def test_factorized_prefill_zero_residual_and_bf16_output():
    """All ranks 0 and all scales 0 give bit-identical outputs (basis-only
    attention); bf16 output is the fp32 result rounded, and repeatable."""
    wl, B, ctx, lens, n, causal = CASES["g4_hd128_ragged"]
    zero = torch.zeros((B, ctx), dtype=torch.uint8)
    a = Factorized(wl, B, ctx, lens, rank_override=zero)
    b = Factorized(wl, B, ctx, lens, scale_zero=True)
    q = datagen.prefill_q(wl, 1, n, batch=B)
    x, y = a.prefill(1, q), b.prefill(1, q)
    assert torch.equal(x, y)
    assert_close(x, a.oracle_prefill(1, q), "bf16", "zero residual")
    h1 = a.prefill(1, q, out_dtype=torch.bfloat16)
    h2 = a.prefill(1, q, out_dtype=torch.bfloat16)
    assert torch.equal(h1, h2)
    assert torch.equal(h1, x.to(torch.bfloat16))


def test_factorized_prefill_row_equals_decode():
    """Row i of a causal chunk equals the factorized decode of the same query
    at seq_len = P_i + 1."""
    import attention_cross_layer_amd as K
    wl, B, ctx, lens, n, causal = CASES["g4_hd128_ragged"]
    d = Factorized(wl, B, ctx, lens)
    q = datagen.prefill_q(wl, 1, n, batch=B)
    got = d.prefill(1, q)
    for i in (0, 31, 64, n - 1):
        pos = [lens[b] - n + i + 1 for b in range(B)]
        seq = torch.tensor(pos, dtype=torch.int32, device="cuda")
        dec = K.kvs_attn_decode(d.plan, d.cache, 1, q[:, i].contiguous().cuda(), seq, max(pos))
        torch.cuda.synchronize()
        diff = float((dec - got[:, i]).abs().max())
        assert diff < 2e-2, (i, diff)


def test_factorized_prefill_full_size_sampled():
    """The 4096-token causal chunk at offset 4096 of an 8192-token prompt on
    the 64K factorized model's heads (32 q / 8 KV, hd 128), batch 1, the launch
    the benchmark times; oracle on sampled query rows (each is attention over
    the rebuilt keys 0..P_i)."""
    T, n = 8192, 4096
    wl = F.with_(n_layers=2, batch=1, ctx=T)
    note(f"[factorized prefill full size] T={T} n={n}")
    d = Factorized(wl, 1, T, [T], dev_gen="cuda", junk=False)
    for layer in (0, 1):
        q = datagen.prefill_q(wl, layer, n, batch=1)
        got = d.prefill(layer, q).double().cpu()
        k, v = d.kv(layer)
        for i in (0, 1, 777, 2048, 4000, 4095):
            P = T - n + i
            ref = A.attend_decode(q[:, i], k, v, [P + 1])
            max_abs, rel = errors(got[:, i], ref)
            note(f"   layer {layer} row {i}: max_abs {max_abs:.2e} rel {rel:.2e}")
            assert max_abs <= 1e-2 and rel <= 5e-3
