"""GPU parity of the factorized write side against the fp64 oracle
(oracle.factorize): the encoder (pair coefficients, int8 residual codes, fp16
scales, placed in the paged layout), the pair basis and the residual
directions (leading singular vectors), and the whole chain feeding decode
attention.  Inputs are seeded rows of strongly correlated layer pairs.

Rounding decisions (a coefficient's bf16 rounding, a scale's fp16 rounding,
a code's round-to-nearest) are taken in fp32 by the kernels and in fp64 by
the oracle, so they may differ where the exact value sits within fp32
accumulation error of a tie: those places are counted and bounded, and
every code is checked against the round-to-nearest bound |y - s d| <= s/2."""
import numpy as np
import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from oracle import factorize as Fz
from tests._gpu_harness import assert_close, errors, note, unpack_factorized

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
F = W["factorized_64k"]


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


class Pair:
    """A two-layer factorized plan (one pair) with correlated rows."""

    def __init__(self, wl, B, ctx, lens):
        self.wl, self.B, self.ctx = wl, B, ctx
        self.lens = list(lens)
        src, w = datagen.share_map(wl)
        cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", B, ctx,
                            kind=K.KVS_FACTORIZED, basis_rank=32, resid_rank_max=16)
        self.src, self.w = src, w
        self.plan = K.kvs_share_plan(cfg, src, w)
        self.cache = K.Cache(self.plan, "cuda")
        for t in (self.cache.ck_pool, self.cache.cv_pool, self.cache.dk_pool, self.cache.dv_pool,
                  self.cache.sk_pool, self.cache.sv_pool, self.cache.rank_pool):
            t.zero_()
        self.ka, self.kb = datagen.correlated_pair_rows(wl, 0, "k", batch=B, ctx=ctx)
        self.va, self.vb = datagen.correlated_pair_rows(wl, 0, "v", batch=B, ctx=ctx)
        self.rank = datagen.token_ranks(wl, batch=B, ctx=ctx)
        self.n_tok = torch.tensor(self.lens, dtype=torch.int32)
        Hkv, hd = wl.n_kv_heads, wl.head_dim
        self.bk_view = self.cache.basis_k.view(torch.bfloat16).view(-1, Hkv, 32, hd)
        self.bv_view = self.cache.basis_v.view(torch.bfloat16).view(-1, Hkv, 32, hd)
        self.uk_view = self.cache.ubasis_k.view(torch.bfloat16).view(-1, Hkv, 16, hd)
        self.uv_view = self.cache.ubasis_v.view(torch.bfloat16).view(-1, Hkv, 16, hd)

    def rows(self, layer):
        return (self.ka, self.va) if layer == 0 else (self.kb, self.vb)

    def oracle_bases(self):
        """Oracle pair basis and residual directions, rounded to bf16 (as stored)."""
        bk = Fz.round_bf16(Fz.pair_basis(self.ka, self.kb, self.lens, 32))
        bv = Fz.round_bf16(Fz.pair_basis(self.va, self.vb, self.lens, 32))
        u = {}
        for l in (0, 1):
            k, v = self.rows(l)
            u[l] = (Fz.round_bf16(Fz.residual_basis(k, self.ka, bk, self.lens, 16)),
                    Fz.round_bf16(Fz.residual_basis(v, self.va, bv, self.lens, 16)))
        return bk, bv, u

    def load_bases(self, bk, bv, u):
        self.bk_view[0].copy_(_bf16(bk))
        self.bv_view[0].copy_(_bf16(bv))
        for l in (0, 1):
            self.uk_view[l].copy_(_bf16(u[l][0]))
            self.uv_view[l].copy_(_bf16(u[l][1]))
        torch.cuda.synchronize()

    def encode(self, lo, hi):
        """Encode positions lo..hi-1 of both layers (owner first)."""
        sp = torch.full((self.B,), lo, dtype=torch.int32).cuda()
        r = self.rank[:, lo:hi].contiguous().cuda()
        ka, va = self.ka[:, lo:hi].contiguous().cuda(), self.va[:, lo:hi].contiguous().cuda()
        K.kvs_encode_factorized(self.plan, self.cache, 0, ka, va, r, sp)
        K.kvs_encode_factorized(self.plan, self.cache, 1, self.kb[:, lo:hi].contiguous().cuda(),
                                self.vb[:, lo:hi].contiguous().cuda(), r, sp, k_owner=ka,
                                v_owner=va)
        torch.cuda.synchronize()


def _count_ulp_mismatch(got, want, ulp_of):
    """Entries that differ, and whether every difference is at most one unit
    in the last place of the stored format."""
    diff = got != want
    if not diff.any():
        return 0, True
    ulp = ulp_of(np.maximum(np.abs(got[diff]), np.abs(want[diff])))
    return int(diff.sum()), bool(np.all(np.abs(got[diff] - want[diff]) <= ulp * 1.0001))


def _ulp_bf16(x):
    return np.ldexp(1.0, np.frexp(x)[1] - 8)


def _ulp_fp16(x):
    return np.maximum(np.ldexp(1.0, np.frexp(x)[1] - 11), 2.0 ** -24)


ENC_CASES = {
    "hd128_g4_two_calls": (F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2), 2, 200, 130),
    "hd64_g8_ragged_tail": (F.with_(n_layers=2, n_q_heads=16, n_kv_heads=2, head_dim=64), 1, 97, 61),
}


@pytest.mark.parametrize("case", list(ENC_CASES))
def test_encoder_matches_oracle(case):
    wl, B, ctx, split = ENC_CASES[case]
    note(f"[encode parity] {case}: B={B} ctx={ctx} split={split} hd={wl.head_dim}")
    p = Pair(wl, B, ctx, [ctx] * B)
    bk, bv, u = p.oracle_bases()
    p.load_bases(bk, bv, u)
    p.encode(0, split)                 # second call starts mid-page
    p.encode(split, ctx)
    for layer in (0, 1):
        ck, cv, dk, dv, sk, sv, rank = unpack_factorized(p.cache, layer, 0, B, ctx, wl.n_kv_heads)
        assert np.array_equal(rank, np.minimum(p.rank.numpy().astype(np.int64), 16))
        x, v = p.rows(layer)
        for side, (xx, xo, basis, ub, c_got, d_got, s_got) in enumerate((
                (x, p.ka, bk, u[layer][0], ck, dk, sk), (v, p.va, bv, u[layer][1], cv, dv, sv))):
            c, y, s, d = Fz.encode(xx, xo, basis, ub, p.rank.numpy())
            what = f"layer {layer} side {'KV'[side]}"
            if layer == 0:
                n_bad, ok = _count_ulp_mismatch(c_got, c, _ulp_bf16)
                note(f"   {what}: coefficients differing by one bf16 ulp: {n_bad} of {c.size}")
                assert ok and n_bad <= max(3, c.size // 1000), what
            n_bad, ok = _count_ulp_mismatch(s_got, s, _ulp_fp16)
            note(f"   {what}: scales differing by one fp16 ulp: {n_bad} of {s.size}")
            assert ok and n_bad <= max(3, s.size // 1000), what
            # every stored code is the round-to-nearest code of the oracle's y
            # under the stored scale, up to fp32 error at ties
            keep = np.arange(16)[None, None, None, :] < p.rank.numpy()[:, :, None, None]
            err = np.abs(y - s_got[..., None] * d_got)
            bound = s_got[..., None] / 2 * (1 + 1e-3) + 1e-6
            assert np.all(np.where(keep, err <= bound, d_got == 0)), what
            assert np.all(np.abs(d_got) <= 127)
            n_code = int(np.sum((d_got != d) & keep))
            note(f"   {what}: codes differing from the oracle's: {n_code} of {int(keep.sum()) * xx.shape[2]}")
            assert n_code <= max(3, int(keep.sum()) * xx.shape[2] // 500), what


def test_encoded_cache_decodes_like_the_oracle():
    """Decode attention over the GPU-encoded cache equals attention over the
    oracle's encoding rebuilt explicitly (both layers, ragged lengths)."""
    wl, B, ctx, split = ENC_CASES["hd128_g4_two_calls"]
    p = Pair(wl, B, ctx, [ctx] * B)
    bk, bv, u = p.oracle_bases()
    p.load_bases(bk, bv, u)
    p.encode(0, ctx)
    lens = [ctx, 123]
    seq = torch.tensor(lens, dtype=torch.int32).cuda()
    for layer in (0, 1):
        x, v = p.rows(layer)
        ck, _, sk, dk = Fz.encode(x, p.ka, bk, u[layer][0], p.rank.numpy())
        cv, _, sv, dv = Fz.encode(v, p.va, bv, u[layer][1], p.rank.numpy())
        kk = A.factorized_kv(ck, bk, sk, dk, u[layer][0], p.rank.numpy())
        vv = A.factorized_kv(cv, bv, sv, dv, u[layer][1], p.rank.numpy())
        q = datagen.decode_q(wl, layer, batch=B)
        got = K.kvs_attn_decode(p.plan, p.cache, layer, q.cuda(), seq, max(lens))
        torch.cuda.synchronize()
        assert_close(got, A.attend_decode(q, kk, vv, lens), "bf16", f"layer {layer}")
        # and the compressed keys stay close to the originals on these rows
        rel = np.linalg.norm(kk - A.f64(x)) / np.linalg.norm(A.f64(x))
        note(f"   layer {layer}: relative key reconstruction error {rel:.3f}")
        assert rel < 0.2


def _basis_checks(got, want, gram_rows, what):
    """Rows of ``got`` (bf16 [Hkv, k, hd]) against the oracle's fp64 leading
    directions ``want``: same order and sign (|cos| of each matching pair near
    1, positive), near-orthonormal, and capturing the oracle's energy."""
    g = got.double().cpu().numpy()
    worst_cos, worst_orth, worst_energy = 1.0, 0.0, 1.0
    for h in range(g.shape[0]):
        cos = np.sum(g[h] * want[h], axis=1) / np.linalg.norm(g[h], axis=1)
        worst_cos = min(worst_cos, float(cos.min()))
        worst_orth = max(worst_orth, float(np.max(np.abs(g[h] @ g[h].T - np.eye(g.shape[1])))))
        rows = gram_rows[h]
        e_got = np.sum((rows @ g[h].T) ** 2)
        e_want = np.sum((rows @ want[h].T) ** 2)
        worst_energy = min(worst_energy, e_got / e_want)
    note(f"   {what}: min cos {worst_cos:.6f}, orthonormality {worst_orth:.2e}, "
         f"energy ratio {worst_energy:.6f}")
    assert worst_cos > 0.999, what
    assert worst_orth < 2e-2, what
    assert worst_energy > 0.999, what


BASIS_CASES = {
    "hd128_ragged": (F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2), 2, 300, [300, 171]),
    "hd64": (F.with_(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64), 1, 256, [256]),
}


@pytest.mark.parametrize("case", list(BASIS_CASES))
def test_pair_basis_matches_oracle(case):
    wl, B, ctx, lens = BASIS_CASES[case]
    note(f"[pair basis parity] {case}: B={B} lens={lens} hd={wl.head_dim}")
    p = Pair(wl, B, ctx, lens)
    Hkv, hd = wl.n_kv_heads, wl.head_dim
    outk = torch.empty((Hkv, 32, hd), dtype=torch.bfloat16, device="cuda")
    outv = torch.empty_like(outk)
    K.kvs_pair_basis(p.plan, p.ka.cuda(), p.va.cuda(), p.kb.cuda(), p.vb.cuda(),
                     p.n_tok.cuda(), outk, outv)
    torch.cuda.synchronize()
    for name, (xa, xb, out) in (("K", (p.ka, p.kb, outk)), ("V", (p.va, p.vb, outv))):
        want = Fz.pair_basis(xa, xb, lens, 32)
        rows = [np.concatenate([A.f64(xa)[b, :lens[b], h] for b in range(B)]
                               + [A.f64(xb)[b, :lens[b], h] for b in range(B)])
                for h in range(Hkv)]
        _basis_checks(out, want, rows, f"pair basis {name}")


@pytest.mark.parametrize("case", list(BASIS_CASES))
def test_residual_basis_matches_oracle(case):
    wl, B, ctx, lens = BASIS_CASES[case]
    note(f"[residual basis parity] {case}: B={B} lens={lens} hd={wl.head_dim}")
    p = Pair(wl, B, ctx, lens)
    Hkv, hd = wl.n_kv_heads, wl.head_dim
    bk = Fz.round_bf16(Fz.pair_basis(p.ka, p.kb, lens, 32))
    bv = Fz.round_bf16(Fz.pair_basis(p.va, p.vb, lens, 32))
    bk_t, bv_t = _bf16(bk).cuda(), _bf16(bv).cuda()
    for layer in (0, 1):
        k, v = p.rows(layer)
        outk = torch.empty((Hkv, 16, hd), dtype=torch.bfloat16, device="cuda")
        outv = torch.empty_like(outk)
        K.kvs_residual_basis(p.plan, k.cuda(), v.cuda(), bk_t, bv_t, p.n_tok.cuda(), outk, outv,
                             k_owner=None if layer == 0 else p.ka.cuda(),
                             v_owner=None if layer == 0 else p.va.cuda())
        torch.cuda.synchronize()
        for name, (x, xo, basis, out) in (("K", (k, p.ka, bk, outk)), ("V", (v, p.va, bv, outv))):
            want = Fz.residual_basis(x, xo, basis, lens, 16)
            e = Fz.residual_rows(x, xo, basis)
            rows = [np.concatenate([e[b, :lens[b], h] for b in range(B)]) for h in range(Hkv)]
            _basis_checks(out, want, rows, f"layer {layer} residual {name}")


def test_gpu_chain_decodes_like_the_oracle_chain():
    """Bases built on the GPU, rows encoded on the GPU, decode on the GPU,
    against the same chain run by the oracle in fp64."""
    wl, B, ctx, lens = BASIS_CASES["hd128_ragged"]
    p = Pair(wl, B, ctx, [ctx] * B)
    Hkv, hd = wl.n_kv_heads, wl.head_dim
    n_tok = torch.full((B,), ctx, dtype=torch.int32).cuda()
    K.kvs_pair_basis(p.plan, p.ka.cuda(), p.va.cuda(), p.kb.cuda(), p.vb.cuda(), n_tok,
                     p.bk_view[0], p.bv_view[0])
    for layer in (0, 1):
        k, v = p.rows(layer)
        K.kvs_residual_basis(p.plan, k.cuda(), v.cuda(), p.bk_view[0], p.bv_view[0], n_tok,
                             p.uk_view[layer], p.uv_view[layer],
                             k_owner=None if layer == 0 else p.ka.cuda(),
                             v_owner=None if layer == 0 else p.va.cuda())
    p.encode(0, ctx)
    bk, bv, u = p.oracle_bases()
    seq = torch.tensor(lens, dtype=torch.int32).cuda()
    for layer in (0, 1):
        x, v = p.rows(layer)
        ck, _, sk, dk = Fz.encode(x, p.ka, bk, u[layer][0], p.rank.numpy())
        cv, _, sv, dv = Fz.encode(v, p.va, bv, u[layer][1], p.rank.numpy())
        kk = A.factorized_kv(ck, bk, sk, dk, u[layer][0], p.rank.numpy())
        vv = A.factorized_kv(cv, bv, sv, dv, u[layer][1], p.rank.numpy())
        q = datagen.decode_q(wl, layer, batch=B)
        got = K.kvs_attn_decode(p.plan, p.cache, layer, q.cuda(), seq, max(lens))
        torch.cuda.synchronize()
        max_abs, rel = errors(got, A.attend_decode(q, kk, vv, lens))
        note(f"   chain layer {layer}: max_abs {max_abs:.2e} rel {rel:.2e}")
        assert max_abs <= 1e-2 and rel <= 5e-3


def test_batched_bases_equal_single_calls():
    """kvs_pair_bases / kvs_residual_bases over several items (one launch
    group, and a workspace that forces groups of one) give bit-identical bases
    to one call per item."""
    wl = F.with_(n_layers=4, n_q_heads=8, n_kv_heads=2)
    B, ctx = 1, 200
    src, w = datagen.share_map(wl)
    cfg = K.make_config(4, 8, 2, 128, "bf16", B, ctx, kind=K.KVS_FACTORIZED, basis_rank=32,
                        resid_rank_max=16)
    plan = K.kvs_share_plan(cfg, src, w)
    n_tok = torch.tensor([ctx - 9], dtype=torch.int32).cuda()
    rows = {}
    for pair in range(2):
        ka, kb = datagen.correlated_pair_rows(wl, pair, "k", batch=B, ctx=ctx)
        va, vb = datagen.correlated_pair_rows(wl, pair, "v", batch=B, ctx=ctx)
        rows[2 * pair], rows[2 * pair + 1] = (ka.cuda(), va.cuda()), (kb.cuda(), vb.cuda())

    def empty(k):
        return [torch.empty((2, k, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    single = [empty(32) for _ in range(2)]
    for pair in range(2):
        (ka, va), (kb, vb) = rows[2 * pair], rows[2 * pair + 1]
        K.kvs_pair_basis(plan, ka, va, kb, vb, n_tok, single[pair][0], single[pair][1])
    item = K.kvs_basis_workspace_size(plan, B, ctx)
    for ws_items in (2, 1):
        ws = torch.empty(item * ws_items, dtype=torch.uint8, device="cuda")
        batched = [empty(32) for _ in range(2)]
        K.kvs_pair_bases(plan, [rows[0][0], rows[2][0]], [rows[0][1], rows[2][1]],
                         [rows[1][0], rows[3][0]], [rows[1][1], rows[3][1]], n_tok,
                         [b[0] for b in batched], [b[1] for b in batched], workspace=ws)
        torch.cuda.synchronize()
        for pair in range(2):
            assert torch.equal(batched[pair][0], single[pair][0])
            assert torch.equal(batched[pair][1], single[pair][1])
    layers = [0, 1, 3]
    owner = {0: None, 1: rows[0], 3: rows[2]}
    single_u = {l: empty(16) for l in layers}
    for l in layers:
        slot = l // 2
        K.kvs_residual_basis(plan, rows[l][0], rows[l][1], single[slot][0], single[slot][1], n_tok,
                             single_u[l][0], single_u[l][1],
                             k_owner=None if owner[l] is None else owner[l][0],
                             v_owner=None if owner[l] is None else owner[l][1])
    for ws_items in (3, 2):
        ws = torch.empty(item * ws_items, dtype=torch.uint8, device="cuda")
        batched_u = {l: empty(16) for l in layers}
        K.kvs_residual_bases(plan, [rows[l][0] for l in layers], [rows[l][1] for l in layers],
                             [single[l // 2][0] for l in layers], [single[l // 2][1] for l in layers],
                             n_tok, [batched_u[l][0] for l in layers], [batched_u[l][1] for l in layers],
                             k_owner=[None if owner[l] is None else owner[l][0] for l in layers],
                             v_owner=[None if owner[l] is None else owner[l][1] for l in layers],
                             workspace=ws)
        torch.cuda.synchronize()
        for l in layers:
            assert torch.equal(batched_u[l][0], single_u[l][0]), (ws_items, l)
            assert torch.equal(batched_u[l][1], single_u[l][1]), (ws_items, l)
