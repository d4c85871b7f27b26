"""GPU parity of the MFMA prefill-chunk kernel against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from tests._gpu_harness import Dense, assert_close, errors, note, TOL_ABS

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS


def _prefill(d, layer, n, causal=True, out_dtype=torch.float32, q=None):
    q = datagen.prefill_q(d.wl, layer, n, batch=d.batch) if q is None else q
    got = K.kvs_attn_prefill_chunk(d.plan, d.cache, layer, q.cuda(), d.seq_len, causal=causal,
                                   out_dtype=out_dtype)
    torch.cuda.synchronize()
    return q, got


CASES = {
    # name: (workload, batch, ctx, lens, n, causal)
    "depthgraft_mixed_ragged": (W["depthgraft"].with_(n_layers=6, dg_stride=2), 2, 320, [300, 200], 130, True),
    "offset0_g4_hd128": (W["cla2_64k"].with_(n_layers=2), 1, 256, [256], 256, True),
    "noncausal_g4_hd128": (W["cla2_64k"].with_(n_layers=2), 2, 200, [200, 77], 64, False),
    "g8_hd64": (W["tinyllama_cla2"].with_(n_layers=2), 2, 520, [500, 333], 100, True),
    "g1_hd64": (W["tinyllama_cla2"].with_(n_layers=2, n_q_heads=4, n_kv_heads=4), 2, 192, [192, 70], 70, True),
    "g2_hd128_mixed": (W["depthgraft"].with_(n_layers=6, dg_stride=2, n_q_heads=16), 1, 150, [150], 33, True),
    "g16_hd128": (W["cla2_64k"].with_(n_layers=2, n_q_heads=16, n_kv_heads=1), 2, 200, [200, 90], 90, True),
    # one query head per KV head and few keys per early row, so single keys
    # dominate rows: the mixed V tile must not be rounded to bf16 alone
    "depthgraft_g1_hd128_few_keys": (W["cla2_64k"].with_(n_layers=6, n_q_heads=1, n_kv_heads=1, share="depthgraft",
                                                         dg_stride=2), 2, 100, [97, 100], 77, True),
    "g32_hd64": (W["tinyllama_cla2"].with_(n_layers=2, n_q_heads=32, n_kv_heads=1), 2, 140, [140, 75], 75, True),
    # the DepthGraft shape (32 q / 8 KV heads, hd 128, owner and mixed layers)
    # at its decode batch of 8, context reduced, ragged lengths
    "depthgraft_b8": (W["depthgraft"].with_(n_layers=6, dg_stride=2), 8, 384,
                      [384, 300, 257, 384, 200, 129, 350, 321], 128, True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_matches_oracle(case):
    wl, B, ctx, lens, n, causal = CASES[case]
    note(f"[prefill parity] {case}: L={wl.n_layers} B={B} lens={lens} n={n} causal={causal} "
         f"Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} hd={wl.head_dim}")
    d = Dense(wl, B, ctx, lens)
    for l in range(wl.n_layers):
        q, got = _prefill(d, l, n, causal)
        ref = A.layer_prefill(d.src.tolist(), d.w.tolist(), l, d.k, d.v, q, lens, causal=causal)
        assert_close(got, ref, "bf16", f"{case} layer {l}")


def test_prefill_bf16_output_and_determinism():
    wl, B, ctx, lens, n, causal = CASES["g8_hd64"]
    d = Dense(wl, B, ctx, lens)
    q, a = _prefill(d, 1, n, out_dtype=torch.bfloat16)
    _, b = _prefill(d, 1, n, out_dtype=torch.bfloat16, q=q)
    assert torch.equal(a, b)
    ref = A.layer_prefill(d.src.tolist(), d.w.tolist(), 1, d.k, d.v, q, lens)
    err = np.abs(a.double().cpu().numpy() - ref)
    assert np.all(err <= TOL_ABS + 2.0 ** -8 * np.abs(ref))


def test_prefill_row_equals_decode():
    """Row i of a causal chunk equals a decode query at seq_len = P_i + 1."""
    wl, B, ctx, lens, n, causal = CASES["depthgraft_mixed_ragged"]
    d = Dense(wl, B, ctx, lens)
    layer = 5                                   # a two-source layer
    q, got = _prefill(d, layer, n)
    for i in (0, 17, n - 1):
        pos = [lens[b] - n + i + 1 for b in range(B)]
        seq = torch.tensor(pos, dtype=torch.int32, device="cuda")
        dec = K.kvs_attn_decode(d.plan, d.cache, layer, q[:, i].contiguous().cuda(), seq, max(pos))
        torch.cuda.synchronize()
        diff = float((dec - got[:, i]).abs().max())
        assert diff < 2e-2, (i, diff)


def test_prefill_full_size_sampled():
    """The 4096-token causal chunk at offset 4096 of an 8192-token prompt,
    batch 1, at the launch configuration the benchmark times; oracle on
    sampled query rows (each is attention over keys 0..P_i)."""
    wl = W["depthgraft"].with_(n_layers=17)
    T, n = 8192, 4096
    note(f"[prefill full size] T={T} n={n}")
    d = Dense(wl, 1, T, [T], kv_device="cuda", nan_fill=False)
    for layer in (8, 16):
        q, got = _prefill(d, layer, n)
        got = got.double().cpu()
        src, w = d.src.tolist(), d.w.tolist()
        kk, vv = A.effective_kv(src[layer], w[layer], d.k, d.v)
        for i in (0, 1, 777, 2048, 4000, 4095):
            P = T - n + i
            ref = A.attend_decode(q[:, i], kk, vv, [P + 1])
            max_abs, rel = errors(got[:, i], ref)
            note(f"   layer {layer} row {i}: max_abs {max_abs:.2e} rel {rel:.2e}")
            assert max_abs <= 1e-2 and rel <= 5e-3


def test_timed_launch_events_on_prefill():
    """The prefill kernel launched with kernel events gives the same output and
    a positive kernel duration."""
    wl, B, ctx, lens, n, causal = CASES["g8_hd64"]
    note("[timed launch] prefill with kernel events")
    d = Dense(wl, B, ctx, lens)
    q, ref = _prefill(d, 0, n)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    K.kvs_time_next_launch(k0, k1)
    _, got = _prefill(d, 0, n, q=q)
    assert torch.equal(got, ref)
    assert k0.elapsed_time(k1) > 0.0
