"""GPU parity of the factorized-cache decode (pair basis + per-layer int8
residual with per-token rank) against the oracle's explicit per-token
reconstruction followed by plain attention."""
import numpy as np
import pytest
import torch

import datagen
from oracle import attention as A
from tests._gpu_harness import Factorized, assert_close, errors, note

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
F = W["factorized_64k"]

CASES = {
    "g4_hd128_junk": (F.with_(n_layers=4, n_q_heads=8, n_kv_heads=2), 2, 300, [300, 150]),
    "g4_hd128_full_heads": (F.with_(n_layers=2), 1, 200, [200]),
    "g8_hd64": (F.with_(n_layers=2, n_q_heads=16, n_kv_heads=2, head_dim=64), 2, 260, [260, 64]),
    "g1_hd64": (F.with_(n_layers=2, n_q_heads=2, n_kv_heads=2, head_dim=64), 2, 129, [129, 1]),
    "g2_hd128": (F.with_(n_layers=2, n_q_heads=4, n_kv_heads=2), 3, 190, [190, 0, 70]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_factorized_decode_matches_oracle(case):
    wl, B, ctx, lens = CASES[case]
    note(f"[factorized parity] {case}: L={wl.n_layers} B={B} lens={lens} Hq={wl.n_q_heads} "
         f"Hkv={wl.n_kv_heads} hd={wl.head_dim}")
    d = Factorized(wl, B, ctx, lens)
    for l in range(wl.n_layers):
        got = d.decode(l)
        torch.cuda.synchronize()
        assert_close(got, d.oracle_decode(l), "bf16", f"{case} layer {l}")


def test_zero_residual_rank_and_scale_agree():
    """All ranks 0 and all scales 0 both remove the residual: the two caches
    give bit-identical outputs (basis-only attention), matching the oracle."""
    wl, B, ctx, lens = CASES["g2_hd128"]
    zero = torch.zeros((B, ctx), dtype=torch.uint8)
    a = Factorized(wl, B, ctx, lens, rank_override=zero)
    b = Factorized(wl, B, ctx, lens, scale_zero=True)
    for l in range(wl.n_layers):
        x, y = a.decode(l), b.decode(l)
        torch.cuda.synchronize()
        assert torch.equal(x, y)
        assert_close(x, a.oracle_decode(l), "bf16", f"zero residual layer {l}")


def test_factorized_split_sweep_and_determinism():
    wl, B, ctx, lens = CASES["g4_hd128_junk"]
    d = Factorized(wl, B, ctx, lens)
    ref = d.oracle_decode(3)
    outs = []
    for s in (1, 2, 3, 5):
        got = d.decode(3, n_splits=s)
        again = d.decode(3, n_splits=s)
        torch.cuda.synchronize()
        assert torch.equal(got, again)
        assert_close(got, ref, "bf16", f"n_splits={s}")
        outs.append(got)


def test_factorized_full_size_sampled():
    """64K-context factorized workload (batch 2, 32 q / 8 KV heads, hd 128),
    one layer pair, library split choice; oracle on every head of sequence 1."""
    wl = F.with_(n_layers=2)
    note(f"[factorized full size] B={wl.batch} ctx={wl.ctx}")
    d = Factorized(wl, wl.batch, wl.ctx, [wl.ctx] * wl.batch, dev_gen="cuda", junk=False)
    for l in (0, 1):
        q = d.q(l)
        got = d.decode(l, q=q).double().cpu()
        torch.cuda.synchronize()
        k, v = d.kv(l, 1, 2)
        ref = A.attend_decode(q[1:2], k, v, [wl.ctx])
        max_abs, rel = errors(got[1:2], ref)
        note(f"   layer {l}: max_abs {max_abs:.2e} rel {rel:.2e}")
        assert max_abs <= 1e-2 and rel <= 5e-3
