"""GPU parity of the token router: the factorized decode's attention
statistics (entropy, peak probability per query) against the oracle's exact
softmax over the rebuilt keys, the rank choice against oracle.router, and
the online loop (encode at a provisional rank, route, encode again)."""
import math

import numpy as np
import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from oracle import factorize as Fz
from oracle import plan as P
from oracle import router as R
from tests._gpu_harness import Factorized, assert_close, note, unpack_factorized

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
F = W["factorized_64k"]

CASES = {
    "g4_hd128_junk": (F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2), 3, 300, [300, 1, 131]),
    "g8_hd64": (F.with_(n_layers=2, n_q_heads=16, n_kv_heads=2, head_dim=64), 2, 260, [260, 64]),
    "g2_top_masked": (F.with_(n_layers=4, n_q_heads=4, n_kv_heads=2, share="pairs_top"), 2, 190,
                      [190, 2]),
}


def _check_stats(got, want, what):
    g = got.double().cpu().numpy()
    err_h = np.abs(g[..., 0] - want[..., 0])
    err_p = np.abs(g[..., 1] - want[..., 1])
    tol_h = 5e-3 * np.maximum(want[..., 0], 1.0)
    tol_p = 5e-3 * np.maximum(want[..., 1], 1e-3)
    note(f"   {what}: entropy err {err_h.max():.2e}, peak err {err_p.max():.2e}")
    assert np.all(err_h <= tol_h) and np.all(err_p <= tol_p), what


@pytest.mark.parametrize("case", list(CASES))
def test_decode_stats_match_oracle(case):
    wl, B, ctx, lens = CASES[case]
    note(f"[router stats parity] {case}: B={B} lens={lens} share={wl.share}")
    d = Factorized(wl, B, ctx, lens)
    for l in range(wl.n_layers):
        q = d.q(l)
        k, _ = d.kv(l)
        excl = P.excludes_current(d.src.tolist(), d.w.tolist(), l)
        want = R.attention_stats(q, k, lens, exclude_current=excl)
        plain = d.decode(l, q=q)
        for s in (1, 3, 0):
            out, st = K.kvs_attn_decode_stats(d.plan, d.cache, l, q.cuda(), d.seq_len, max(lens),
                                              n_splits=s)
            torch.cuda.synchronize()
            if s == 0:
                assert torch.equal(out, plain), "statistics change the output"
            assert_close(out, d.oracle_decode(l, q=q), "bf16", f"{case} layer {l} n_splits={s}")
            _check_stats(st, want, f"{case} layer {l} n_splits={s}")


def test_dense_plan_rejects_statistics():
    wl = W["tinyllama_cla2"].with_(n_layers=2)
    src, w = datagen.share_map(wl)
    cfg = K.make_config(2, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", 1, 64)
    plan = K.kvs_share_plan(cfg, src, w)
    cache = K.Cache(plan, "cuda")
    q = datagen.decode_q(wl, 0, batch=1).cuda()
    with pytest.raises(K.KvsError) as e:
        K.kvs_attn_decode_stats(plan, cache, 0, q, torch.tensor([64], dtype=torch.int32).cuda(), 64)
    assert e.value.status == K.KVS_ERR_UNSUPPORTED


def _router(ef=0.3, ed=0.7, pf=0.95, rf=16, rm=8, rd=0):
    return K.kvs_router(ef, ed, pf, rf, rm, rd)


def test_route_ranks_match_oracle():
    """Seeded statistics for 300 sequences, two sets, 8 heads, ragged key
    counts: ranks equal the oracle's wherever its mean normalized entropy is
    not within 1e-5 of a threshold."""
    wl = F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2)
    src, w = datagen.share_map(wl)
    B = 300
    cfg = K.make_config(2, 8, 2, 128, "bf16", B, 64, kind=K.KVS_FACTORIZED, basis_rank=32,
                        resid_rank_max=16)
    plan = K.kvs_share_plan(cfg, src, w)
    g = np.random.default_rng(4)
    n_keys = g.integers(0, 5000, B)
    n_keys[:3] = (0, 1, 2)
    ln = np.log(np.maximum(n_keys, 2))
    st = np.zeros((2, B, 8, 2), dtype=np.float32)
    # per-sequence level in [0, 1) plus per-head spread: the mean spans all three ranks
    level = g.uniform(0, 1, (1, B, 1))
    spread = np.clip(level + g.uniform(-0.1, 0.1, (2, B, 8)), 0, 1)
    st[..., 0] = (spread * ln[None, :, None]).astype(np.float32)
    st[..., 1] = g.uniform(0, 1, (2, B, 8)) ** 4
    for pf in (0.95, 0.5, 2.0):
        r = _router(pf=pf)
        got = K.kvs_route_ranks(plan, torch.from_numpy(st).cuda(),
                                torch.from_numpy(n_keys.astype(np.int32)).cuda(), r)
        torch.cuda.synchronize()
        want, h, _ = R.route_ranks(st.astype(np.float64), n_keys, 0.3, 0.7, pf, 16, 8, 0)
        near = (np.abs(h - 0.3) < 1e-5) | (np.abs(h - 0.7) < 1e-5)
        got = got.cpu().numpy().astype(np.int64)
        assert np.array_equal(got[~near], want[~near]), pf
        note(f"   peak threshold {pf}: ranks {np.bincount(got, minlength=17)[[0, 8, 16]]} (0/8/16), "
             f"{int(near.sum())} near a threshold")
    # ranks clamp to [0, Rmax]
    got = K.kvs_route_ranks(plan, torch.from_numpy(st).cuda(),
                            torch.from_numpy(n_keys.astype(np.int32)).cuda(), _router(rf=99, rd=-5))
    assert int(got.max()) <= 16


def test_routed_rank_reencodes_the_current_token():
    """One decode step of the online loop on a correlated pair: the current
    token is encoded at the top rank, layer 0's decode yields statistics, the
    router picks a rank, and the token is encoded again at that rank; the
    stored rank, and decode over the cache, then match the oracle built with
    the routed rank."""
    from tests.test_gpu_encode import Pair
    wl = F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2)
    B, T = 2, 130                                    # current token: position 129
    p = Pair(wl, B, T, [T] * B)
    bk, bv, u = p.oracle_bases()
    p.load_bases(bk, bv, u)
    rank = p.rank.clone()
    rank[:, T - 1] = 16
    p.rank = rank
    p.encode(0, T)
    q0 = datagen.decode_q(wl, 0, batch=B)
    seq = torch.full((B,), T, dtype=torch.int32).cuda()
    _, st = K.kvs_attn_decode_stats(p.plan, p.cache, 0, q0.cuda(), seq, T)
    # thresholds around the measured entropy so that the two sequences differ
    h = st[..., 0].double().mean(dim=1).cpu().numpy() / math.log(T)
    mid = float(np.mean(h))
    r = _router(ef=min(h) - 1e-3, ed=mid, pf=2.0)
    routed = K.kvs_route_ranks(p.plan, st, seq, r)
    torch.cuda.synchronize()
    want, hh, _ = R.route_ranks(st.double().cpu().numpy(), [T] * B, min(h) - 1e-3, mid, 2.0, 16, 8, 0)
    assert np.array_equal(routed.cpu().numpy().astype(np.int64), want)
    note(f"   routed ranks {routed.cpu().tolist()} from normalized entropies {h.round(4).tolist()}")
    rank[:, T - 1] = routed.cpu()
    p.rank = rank
    p.encode(T - 1, T)                              # encode the current token again
    for layer in (0, 1):
        ck, cv, dk, dv, sk, sv, stored = unpack_factorized(p.cache, layer, 0, B, T, wl.n_kv_heads)
        assert np.array_equal(stored[:, T - 1], routed.cpu().numpy().astype(np.int64))
        x, v = p.rows(layer)
        c1, _, s1, d1 = Fz.encode(x, p.ka, bk, u[layer][0], rank.numpy())
        c2, _, s2, d2 = Fz.encode(v, p.va, bv, u[layer][1], rank.numpy())
        kk = A.factorized_kv(c1, bk, s1, d1, u[layer][0], rank.numpy())
        vv = A.factorized_kv(c2, bv, s2, d2, u[layer][1], rank.numpy())
        q = datagen.decode_q(wl, layer, batch=B)
        got = K.kvs_attn_decode(p.plan, p.cache, layer, q.cuda(), seq, T)
        torch.cuda.synchronize()
        assert_close(got, A.attend_decode(q, kk, vv, [T] * B), "bf16", f"layer {layer}")


def test_full_size_stats_sampled():
    """64K-context factorized workload (batch 2, 32 q / 8 KV heads), one
    layer pair, library split choice: statistics of every head of sequence 1
    against the oracle."""
    wl = F.with_(n_layers=2)
    note(f"[router full size] B={wl.batch} ctx={wl.ctx}")
    d = Factorized(wl, wl.batch, wl.ctx, [wl.ctx] * wl.batch, dev_gen="cuda", junk=False)
    for l in (0, 1):
        q = d.q(l)
        _, st = K.kvs_attn_decode_stats(d.plan, d.cache, l, q.cuda(), d.seq_len, wl.ctx)
        torch.cuda.synchronize()
        k, _ = d.kv(l, 1, 2)
        want = R.attention_stats(q[1:2], k, [wl.ctx])
        _check_stats(st[1:2], want, f"layer {l}")
