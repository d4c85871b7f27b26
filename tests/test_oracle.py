"""Pins for the fp64 oracle: closed forms, a library routine, invariants and
brute force.  None of these compares the oracle with itself on the same
formula; each would fail under a plausible mistake in the oracle (checked in
``test_planted_mistakes_are_caught``)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import datagen
from oracle import attention as A
from oracle import plan as P


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


# ----------------------------------------------------------------------------
# closed forms (hand-derived fixtures)
# ----------------------------------------------------------------------------

def check_two_key(golden, attend_decode=A.attend_decode):
    q = np.array(golden["q"])[None, None, :]
    k = np.array(golden["k"])[None, :, None, :]
    v = np.array(golden["v"])[None, :, None, :]
    out = attend_decode(q, k, v, [2])
    return np.max(np.abs(out[0, 0] - np.array(golden["out"])))


def test_golden_two_key_softmax(golden_dir):
    assert check_two_key(_load(golden_dir, "two_key_softmax.json")) < 1e-12


def check_causal(golden, attend_prefill=A.attend_prefill):
    T, n = golden["seq_len"], golden["n"]
    v = np.array(golden["v"])[None, :, None, :]
    k = np.zeros_like(v)
    q = np.zeros((1, n, 1, v.shape[-1]))
    out = attend_prefill(q, k, v, [T], causal=True)
    return np.max(np.abs(out[0, :, 0, :] - np.array(golden["out"])))


def test_golden_causal_offset(golden_dir):
    assert check_causal(_load(golden_dir, "causal_offset.json")) < 1e-12


def check_factorized_token(golden, factorized_kv=A.factorized_kv):
    c = np.array(golden["c"])[None, None, None, :]
    basis = np.array(golden["basis"])[None]
    u = np.array(golden["u"])[None]
    s = np.array([[[golden["scale"]]]])
    d = np.array(golden["d"])[None, None, None, :]
    r = np.array([[golden["rank"]]])
    k = factorized_kv(c, basis, s, d, u, r)
    return np.max(np.abs(k[0, 0, 0] - np.array(golden["k"])))


def test_golden_factorized_token(golden_dir):
    assert check_factorized_token(_load(golden_dir, "factorized_token.json")) == 0.0


def check_gqa_grouping(attend_decode=A.attend_decode):
    """Hq=4, Hkv=2: every value row of KV head g is e_g, so query head h must
    return e_{h // 2} whatever the scores."""
    B, T, Hkv, hd = 1, 5, 2, 4
    k = _rand((B, T, Hkv, hd), 7).numpy()
    v = np.zeros((B, T, Hkv, hd))
    v[:, :, 0, 0] = 1.0
    v[:, :, 1, 1] = 1.0
    q = _rand((B, 4, hd), 8).numpy()
    out = attend_decode(q, k, v, [T])
    want = np.zeros((4, hd))
    for h in range(4):
        want[h, h // 2] = 1.0
    return np.max(np.abs(out[0] - want))


def test_gqa_grouping_consecutive():
    assert check_gqa_grouping() < 1e-12


def test_equal_keys_give_mean_of_values():
    B, T, Hq, Hkv, hd = 2, 9, 4, 2, 8
    k = np.broadcast_to(_rand((1, 1, Hkv, hd), 1).numpy(), (B, T, Hkv, hd)).copy()
    v = _rand((B, T, Hkv, hd), 2).numpy()
    q = _rand((B, Hq, hd), 3).numpy() * 5
    lens = [T, 4]
    out = A.attend_decode(q, k, v, lens)
    for b in range(B):
        for h in range(Hq):
            assert np.allclose(out[b, h], v[b, :lens[b], h // 2].mean(axis=0), atol=1e-13)


def test_single_key_returns_its_value():
    B, T, Hq, Hkv, hd = 1, 6, 2, 1, 16
    k = _rand((B, T, Hkv, hd), 4).numpy()
    v = _rand((B, T, Hkv, hd), 5).numpy()
    q = _rand((B, Hq, hd), 6).numpy()
    out = A.attend_decode(q, k, v, [1])
    assert np.allclose(out[0, :, :], v[0, 0, 0][None, :], atol=1e-15)


def test_dominant_key_takes_all_weight():
    B, T, Hq, Hkv, hd = 1, 32, 1, 1, 16
    k = _rand((B, T, Hkv, hd), 9).numpy() * 0.01
    q = np.ones((B, Hq, hd))
    k[0, 17, 0] = 100.0
    v = _rand((B, T, Hkv, hd), 10).numpy()
    out = A.attend_decode(q, k, v, [T])
    assert np.allclose(out[0, 0], v[0, 17, 0], atol=1e-12)


# ----------------------------------------------------------------------------
# library routine: PyTorch SDPA in float64 with explicitly repeated KV heads
# ----------------------------------------------------------------------------

def _sdpa(q, k, v, G, mask=None, is_causal=False):
    """q [B, n, Hq, hd], k/v [B, T, Hkv, hd] (float64 torch) -> [B, n, Hq, hd]."""
    qt = q.permute(0, 2, 1, 3)
    kt = k.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = v.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                         is_causal=is_causal)
    return o.permute(0, 2, 1, 3)


@pytest.mark.parametrize("Hq,Hkv,hd", [(4, 2, 64), (32, 4, 64), (8, 8, 32), (32, 1, 64)])
def test_decode_matches_sdpa(Hq, Hkv, hd):
    B, T = 3, 70
    q = _rand((B, Hq, hd), 11)
    k = _rand((B, T, Hkv, hd), 12)
    v = _rand((B, T, Hkv, hd), 13)
    lens = [T, 1, 33]
    out = A.attend_decode(q.numpy(), k.numpy(), v.numpy(), lens)
    for b, L in enumerate(lens):
        ref = _sdpa(q[b:b + 1, None], k[b:b + 1, :L], v[b:b + 1, :L], Hq // Hkv)
        assert np.max(np.abs(out[b] - ref[0, 0].numpy())) < 1e-12


def test_prefill_matches_sdpa_causal_and_full():
    B, n, Hq, Hkv, hd = 2, 7, 4, 2, 16
    q = _rand((B, n, Hq, hd), 21)
    k = _rand((B, 19, Hkv, hd), 22)
    v = _rand((B, 19, Hkv, hd), 23)
    # offset 0: the chunk is the whole sequence -> library causal mask
    out0 = A.attend_prefill(q.numpy(), k[:, :n].numpy(), v[:, :n].numpy(), [n, n], causal=True)
    ref0 = _sdpa(q, k[:, :n], v[:, :n], Hq // Hkv, is_causal=True)
    assert np.max(np.abs(out0 - ref0.numpy())) < 1e-12
    # offset 12: query i at position 12 + i sees keys 0..12+i (bool mask = allowed)
    T = 19
    mask = torch.ones(n, T, dtype=torch.bool).tril(diagonal=T - n)
    outc = A.attend_prefill(q.numpy(), k.numpy(), v.numpy(), [T, T], causal=True)
    refc = _sdpa(q, k, v, Hq // Hkv, mask=mask)
    assert np.max(np.abs(outc - refc.numpy())) < 1e-12
    # non-causal: every query sees the whole sequence
    outf = A.attend_prefill(q.numpy(), k.numpy(), v.numpy(), [T, T], causal=False)
    reff = _sdpa(q, k, v, Hq // Hkv)
    assert np.max(np.abs(outf - reff.numpy())) < 1e-12


def test_prefill_row_equals_decode_at_its_position():
    B, n, Hq, Hkv, hd, T = 2, 5, 4, 2, 8, 13
    q = _rand((B, n, Hq, hd), 31).numpy()
    k = _rand((B, T, Hkv, hd), 32).numpy()
    v = _rand((B, T, Hkv, hd), 33).numpy()
    out = A.attend_prefill(q, k, v, [T, T], causal=True)
    for i in range(n):
        d = A.attend_decode(q[:, i], k, v, [T - n + i + 1] * B)
        assert np.max(np.abs(out[:, i] - d)) < 1e-13


# ----------------------------------------------------------------------------
# brute force: pure-Python loops on tiny shapes
# ----------------------------------------------------------------------------

def _brute_decode(q, k, v, lens):
    B, Hq, hd = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    out = [[[0.0] * hd for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            zs = []
            for t in range(lens[b]):
                zs.append(sum(q[b][h][d] * k[b][t][g][d] for d in range(hd)) / math.sqrt(hd))
            mx = max(zs)
            ws = [math.exp(z - mx) for z in zs]
            den = math.fsum(ws)
            for d in range(hd):
                out[b][h][d] = math.fsum(ws[t] * v[b][t][g][d] for t in range(lens[b])) / den
    return out


def test_brute_force_decode_tiny_workload():
    wl = datagen.WORKLOADS["tiny_cla2"].with_(ctx=24)
    k, v = datagen.owner_kv(wl, 0)
    q = datagen.decode_q(wl, 1)
    lens = [24]
    got = A.attend_decode(q, k, v, lens)
    want = np.array(_brute_decode(A.f64(q).tolist(), A.f64(k).tolist(), A.f64(v).tolist(), lens))
    assert np.max(np.abs(got - want)) < 1e-12


def test_brute_force_factorized_tiny():
    wl = datagen.WORKLOADS["factorized_64k"].with_(batch=2, ctx=10, n_kv_heads=2,
                                                    n_q_heads=4, head_dim=16,
                                                    basis_rank=4, resid_rank_max=3,
                                                    rank16_frac=0.3)
    rank = datagen.token_ranks(wl, ranks=(0, 1, 3))
    ck, _ = datagen.pair_coeffs(wl, 0)
    bk, _ = datagen.pair_basis(wl, 0)
    uk, _ = datagen.layer_residual_basis(wl, 1)
    dk, _, sk, _ = datagen.layer_residual(wl, 1, rank, junk_beyond_rank=True)
    got = A.factorized_kv(ck, bk, sk, dk, uk, rank)
    c, B_, s, d, u = (A.f64(x) for x in (ck, bk, sk, dk, uk))
    for b in range(2):
        for t in range(10):
            r = int(rank[b, t])
            for g in range(2):
                for e in range(16):
                    want = math.fsum(c[b, t, g, i] * B_[g, i, e] for i in range(4))
                    want += s[b, t, g] * math.fsum(d[b, t, g, j] * u[g, j, e] for j in range(r))
                    assert abs(got[b, t, g, e] - want) < 1e-12


# ----------------------------------------------------------------------------
# map indirection invariants
# ----------------------------------------------------------------------------

def _small_dense(share, L, seed_shift=0):
    wl = datagen.WORKLOADS["depthgraft" if share == "depthgraft" else "tinyllama_cla2"]
    wl = wl.with_(n_layers=L, batch=2, ctx=40, n_q_heads=8, n_kv_heads=2, head_dim=16,
                  seed=wl.seed + seed_shift, dg_stride=2)
    src, w = datagen.share_map(wl)
    ok = datagen.owner_layers(src)
    kk, vv = {}, {}
    for l in ok:
        kk[l], vv[l] = datagen.owner_kv(wl, l)
    return wl, src, w, kk, vv


@pytest.mark.parametrize("share,L", [("cla2", 6), ("depthgraft", 6)])
def test_map_equals_identity_on_materialised_cache(share, L):
    """oracle(map) == oracle(identity map) on a cache where each layer's slot
    holds the w-mix of its sources, materialised by hand in float64."""
    wl, src, w, kk, vv = _small_dense(share, L)
    lens = [40, 17]
    ident_k, ident_v = {}, {}
    for l in range(L):
        acc_k = np.zeros(A.f64(kk[next(iter(kk))]).shape)
        acc_v = np.zeros_like(acc_k)
        for j in range(2):
            s = int(src[l, j])
            if s >= 0:
                acc_k += float(w[l, j]) * A.f64(kk[s])
                acc_v += float(w[l, j]) * A.f64(vv[s])
        ident_k[l], ident_v[l] = acc_k, acc_v
    isrc = [[l, -1] for l in range(L)]
    iw = [[1.0, 0.0] for _ in range(L)]
    for l in range(L):
        q = datagen.decode_q(wl, l)
        a = A.layer_decode(src.tolist(), w.tolist(), l, kk, vv, q, lens)
        b = A.layer_decode(isrc, iw, l, ident_k, ident_v, q, lens)
        assert np.max(np.abs(a - b)) < 1e-12


def test_layers_sharing_a_source_with_same_query_agree():
    wl, src, w, kk, vv = _small_dense("cla2", 6)
    q = datagen.decode_q(wl, 0)
    lens = [40, 3]
    a = A.layer_decode(src.tolist(), w.tolist(), 4, kk, vv, q, lens)
    b = A.layer_decode(src.tolist(), w.tolist(), 5, kk, vv, q, lens)
    assert np.array_equal(a, b)
    c = A.layer_decode(src.tolist(), w.tolist(), 3, kk, vv, q, lens)
    assert np.max(np.abs(a - c)) > 1e-3   # a different source gives a different answer


def test_depthgraft_mix_special_cases():
    wl, src, w, kk, vv = _small_dense("depthgraft", 6)
    src = src.tolist()
    lens = [40, 25]
    l = 5                    # reads layers 3 and 1
    assert src[l] == [3, 1]
    q = datagen.decode_q(wl, l)
    only_near = A.layer_decode([[s, -1] for s, _ in src], [[1.0, 0.0]] * 6, 3, kk, vv, q, lens)
    only_far = A.layer_decode([[s, -1] for s, _ in src], [[1.0, 0.0]] * 6, 1, kk, vv, q, lens)
    w1 = [[1.0, 0.0]] * 6
    w1[l] = [1.0, 0.0]
    assert np.array_equal(A.layer_decode(src, w1, l, kk, vv, q, lens), only_near)
    w0 = [[1.0, 0.0]] * 6
    w0[l] = [0.0, 1.0]
    assert np.array_equal(A.layer_decode(src, w0, l, kk, vv, q, lens), only_far)
    # two identical sources: any split of weight 1 is a single source
    kk2, vv2 = dict(kk), dict(vv)
    kk2[1], vv2[1] = kk[3], vv[3]
    wm = [[1.0, 0.0]] * 6
    wm[l] = [0.375, 0.625]
    assert np.max(np.abs(A.layer_decode(src, wm, l, kk2, vv2, q, lens) - only_near)) < 1e-12


def test_attention_is_linear_in_values():
    B, T, Hq, Hkv, hd = 2, 21, 4, 2, 8
    q = _rand((B, Hq, hd), 41).numpy()
    k = _rand((B, T, Hkv, hd), 42).numpy()
    v1 = _rand((B, T, Hkv, hd), 43).numpy()
    v2 = _rand((B, T, Hkv, hd), 44).numpy()
    a, b = 0.3, 0.7
    lhs = A.attend_decode(q, k, a * v1 + b * v2, [T, 9])
    rhs = a * A.attend_decode(q, k, v1, [T, 9]) + b * A.attend_decode(q, k, v2, [T, 9])
    assert np.max(np.abs(lhs - rhs)) < 1e-13


# ----------------------------------------------------------------------------
# factorized cache
# ----------------------------------------------------------------------------

def _fact_small(junk=False):
    wl = datagen.WORKLOADS["factorized_64k"].with_(batch=2, ctx=50, n_kv_heads=2,
                                                    n_q_heads=8, head_dim=64)
    rank = datagen.token_ranks(wl)
    ck, cv = datagen.pair_coeffs(wl, 0)
    bk, bv = datagen.pair_basis(wl, 0)
    uk, uv = datagen.layer_residual_basis(wl, 1)
    dk, dv, sk, sv = datagen.layer_residual(wl, 1, rank, junk_beyond_rank=junk)
    return wl, rank, ck, cv, bk, bv, uk, uv, dk, dv, sk, sv


def test_factorized_unit_basis_matches_sdpa():
    """Basis rows e_0..e_31 and residual rows e_32..e_47 make K exactly
    [c, s*d (first r codes), 0...]; attention over that explicit K must match
    the library SDPA."""
    wl, rank, ck, cv, bk, bv, uk, uv, dk, dv, sk, sv = _fact_small(junk=True)
    hd, R, Rm = 64, 32, 16
    eye = torch.eye(hd, dtype=torch.float64)
    basis = eye[:R].expand(2, R, hd)
    u = eye[R:R + Rm].expand(2, Rm, hd)
    k = A.factorized_kv(ck, basis, sk, dk, u, rank)
    v = A.factorized_kv(cv, basis, sv, dv, u, rank)
    used = (torch.arange(Rm)[None, None, :] < rank[:, :, None].long()).double()
    k_exp = torch.zeros(2, 50, 2, hd, dtype=torch.float64)
    k_exp[..., :R] = ck.double()
    k_exp[..., R:R + Rm] = sk.double()[..., None] * dk.double() * used[:, :, None, :]
    v_exp = torch.zeros_like(k_exp)
    v_exp[..., :R] = cv.double()
    v_exp[..., R:R + Rm] = sv.double()[..., None] * dv.double() * used[:, :, None, :]
    assert np.array_equal(k, k_exp.numpy()) and np.array_equal(v, v_exp.numpy())
    q = datagen.decode_q(wl, 1).double()
    out = A.attend_decode(q, k, v, [50, 50])
    ref = _sdpa(q[:, None], k_exp, v_exp, 4)[:, 0]
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_factorized_zero_residual_is_basis_only():
    wl, rank, ck, cv, bk, bv, uk, uv, dk, dv, sk, sv = _fact_small()
    zero_rank = torch.zeros_like(rank)
    k = A.factorized_kv(ck, bk, sk, dk, uk, zero_rank)
    assert np.max(np.abs(k - np.einsum("btgi,gid->btgd", A.f64(ck), A.f64(bk)))) < 1e-12
    k2 = A.factorized_kv(ck, bk, torch.zeros_like(sk), dk, uk, rank)
    assert np.array_equal(k, k2)


def test_factorized_ranks_follow_the_recipe():
    wl = datagen.WORKLOADS["factorized_64k"].with_(batch=2, ctx=65536)
    r = datagen.token_ranks(wl)
    for b in range(2):
        counts = torch.bincount(r[b].long(), minlength=17)
        assert int(counts[16]) == 6554 and int(counts[8]) == 29491 and int(counts[0]) == 29491


# ----------------------------------------------------------------------------
# planner semantics
# ----------------------------------------------------------------------------

def test_plan_reduction_factors_from_the_pages():
    # CLA2 halves the cache (CLA page, Key Results / Abstract)
    src, w = datagen.share_map(datagen.WORKLOADS["tinyllama_cla2"])
    assert P.check(src.tolist(), w.tolist()) == P.OK
    assert len(P.owner_layers(src.tolist(), w.tolist())) == 11
    assert P.cache_fraction(src.tolist(), w.tolist()) == 0.5
    # DepthGraft cuts roughly one third (DepthGraft page, Abstract)
    src, w = datagen.share_map(datagen.WORKLOADS["depthgraft"])
    assert P.check(src.tolist(), w.tolist()) == P.OK
    assert P.owner_layers(src.tolist(), w.tolist()) == list(range(16))
    assert abs(P.cache_fraction(src.tolist(), w.tolist()) - 2 / 3) < 1e-12
    assert P.last_owner_layer(src.tolist(), w.tolist()) == 15
    srcs = P.layer_sources(src.tolist(), w.tolist(), 20)
    assert [s for s, _, _ in srcs] == [12, 4] and [sl for _, sl, _ in srcs] == [12, 4]
    assert abs(srcs[0][2] + srcs[1][2] - 1.0) < 1e-6


def test_plan_slot_numbering_ascending():
    src = [[0, -1], [0, -1], [2, -1], [2, -1], [4, -1]]
    w = [[1.0, 0.0]] * 5
    assert P.slots(src, w) == {0: 0, 2: 1, 4: 2}


@pytest.mark.parametrize("src,w,want", [
    ([[0, -1], [0, -1]], [[1.0, 0], [1.0, 0]], P.OK),
    ([[0, -1], [2, -1]], [[1.0, 0], [1.0, 0]], P.ERR_MAP),          # out of range
    ([[0, -1], [1, -1], [1, -1]], [[1.0, 0], [0.5, 0], [1.0, 0]], P.ERR_MAP),  # self row w != 1
    ([[0, -1], [0, -1], [1, -1]], [[1.0, 0]] * 3, P.ERR_NOT_SOURCE),  # chain
    ([[1, -1], [1, -1]], [[1.0, 0], [1.0, 0]], P.OK),               # source above reader (top)
    ([[1, -1], [1, -1], [1, -1]], [[1.0, 0]] * 3, P.OK),             # middle: 0 and 2 read 1
    ([[2, -1], [2, -1], [1, -1]], [[1.0, 0]] * 3, P.ERR_NOT_SOURCE), # 2 reads a non-owner
    ([[0, -1], [0, -1]], [[1.0, 0], [float("nan"), 0]], P.ERR_MAP),
    ([[0, -1], [1, 0]], [[1.0, 0], [0.5, 0.5]], P.ERR_MAP),           # self + other
])
def test_plan_rules(src, w, want):
    assert P.check(src, w) == want


# ----------------------------------------------------------------------------
# top / middle configurations: diagonal masking ("A Systematic Study of
# Cross-Layer KV Sharing for Efficient LLM Inference", TL;DR)
# ----------------------------------------------------------------------------

def check_strict_prefill(attend_prefill=A.attend_prefill):
    """Strict causal prefill (query at P sees keys j < P) against the library
    SDPA with the explicit strict mask, at offset 0 (first row: no key,
    zeros) and at offset 12."""
    B, n, Hq, Hkv, hd, T = 2, 7, 4, 2, 16, 19
    q = _rand((B, n, Hq, hd), 61)
    k = _rand((B, T, Hkv, hd), 62)
    v = _rand((B, T, Hkv, hd), 63)
    err = 0.0
    mask = torch.ones(n, T, dtype=torch.bool).tril(diagonal=T - n - 1)
    out = attend_prefill(q.numpy(), k.numpy(), v.numpy(), [T, T], causal=True, exclude_current=True)
    err = max(err, float(np.max(np.abs(out - _sdpa(q, k, v, Hq // Hkv, mask=mask).numpy()))))
    mask0 = torch.ones(n, n, dtype=torch.bool).tril(diagonal=-1)
    out0 = attend_prefill(q.numpy(), k[:, :n].numpy(), v[:, :n].numpy(), [n, n], causal=True,
                          exclude_current=True)
    ref0 = _sdpa(q[:, 1:], k[:, :n], v[:, :n], Hq // Hkv, mask=mask0[1:]).numpy()
    err = max(err, float(np.max(np.abs(out0[:, 1:] - ref0))))
    err = max(err, float(np.max(np.abs(out0[:, 0]))))            # position 0 sees nothing
    return err


def test_strict_prefill_matches_sdpa_with_strict_mask():
    assert check_strict_prefill() < 1e-12


def test_top_decode_skips_the_current_position():
    """A layer reading a source above it: at seq_len T its query equals a
    plain decode over keys 0..T-2 (a different routine: attend over an
    explicitly shortened cache), and T = 1 gives zeros."""
    B, Hq, Hkv, hd, T = 2, 4, 2, 16, 9
    q = _rand((B, Hq, hd), 71)
    k = _rand((B, T, Hkv, hd), 72)
    v = _rand((B, T, Hkv, hd), 73)
    src = [[1, -1], [1, -1]]
    w = [[1.0, 0.0], [1.0, 0.0]]
    top = A.layer_decode(src, w, 0, {1: k.numpy()}, {1: v.numpy()}, q.numpy(), [T, T])
    ref = _sdpa(q[:, None], k[:, :T - 1], v[:, :T - 1], Hq // Hkv)[:, 0].numpy()
    assert np.max(np.abs(top - ref)) < 1e-12
    own = A.layer_decode(src, w, 1, {1: k.numpy()}, {1: v.numpy()}, q.numpy(), [T, T])
    assert np.max(np.abs(own - _sdpa(q[:, None], k, v, Hq // Hkv)[:, 0].numpy())) < 1e-12
    assert np.all(A.layer_decode(src, w, 0, {1: k.numpy()}, {1: v.numpy()}, q.numpy(), [1, 1]) == 0)
    assert P.excludes_current(src, w, 0) and not P.excludes_current(src, w, 1)


def test_top_cla2_halves_the_cache():
    src = [[1, -1], [1, -1], [3, -1], [3, -1]]
    w = [[1.0, 0.0]] * 4
    assert P.check(src, w) == P.OK
    assert P.cache_fraction(src, w) == 0.5
    assert [P.excludes_current(src, w, l) for l in range(4)] == [True, False, True, False]


# ----------------------------------------------------------------------------
# the pins catch planted mistakes
# ----------------------------------------------------------------------------

def test_planted_mistakes_are_caught(golden_dir, monkeypatch):
    two = _load(golden_dir, "two_key_softmax.json")
    cau = _load(golden_dir, "causal_offset.json")
    fac = _load(golden_dir, "factorized_token.json")

    def wrong_scale(q, k, v, seq_len, scale=None):
        return A.attend_decode(q, k, v, seq_len, scale=1.0 / q.shape[-1])

    assert check_two_key(two, wrong_scale) > 0.1

    def wrong_group(q, k, v, seq_len, scale=None):  # h % Hkv instead of h // G
        q = A.f64(q)
        Hq, Hkv = q.shape[1], A.f64(k).shape[2]
        perm = [h % Hkv * (Hq // Hkv) + h // Hkv for h in range(Hq)]
        return A.attend_decode(q[:, perm], k, v, seq_len)[:, np.argsort(perm)]

    assert check_gqa_grouping(wrong_group) > 0.5

    def strict_causal(q, k, v, seq_len, causal=True, scale=None):  # j < P instead of j <= P
        out = A.attend_prefill(q, k, v, [s - 1 for s in seq_len], causal=True)
        return out

    assert check_causal(cau, strict_causal) > 0.1

    def inclusive_diagonal(q, k, v, seq_len, causal=True, scale=None, exclude_current=False):
        return A.attend_prefill(q, k, v, seq_len, causal=causal)    # masking ignored

    assert check_strict_prefill(inclusive_diagonal) > 0.1

    def rank_off_by_one(c, basis, scale, d, u, rank):
        return A.factorized_kv(c, basis, scale, d, u, np.asarray(rank) + 1)

    assert check_factorized_token(fac, rank_off_by_one) > 1.0

    def swapped_b_u(c, basis, scale, d, u, rank):
        return A.factorized_kv(c, u, scale, d, basis, rank)

    assert check_factorized_token(fac, swapped_b_u) > 1.0
