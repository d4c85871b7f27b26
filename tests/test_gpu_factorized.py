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


def test_factorized_append_layout_bit_exact():
    """Pool bytes after two appends (the second starting mid-page, so granule
    offsets come partly from stored ranks) equal the documented layout:
    cK chunk-major, cV quad-interleaved, rank-packed code granules with zeros
    past each rank, meta = rank | granule offset << 8."""
    wl = F.with_(n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64)
    B, ctx, n1, n2 = 2, 192, 100, 70
    import attention_cross_layer_amd as K
    src, w = datagen.share_map(wl)
    cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", B, ctx,
                        kind=K.KVS_FACTORIZED, basis_rank=32, resid_rank_max=16)
    plan = K.kvs_share_plan(cfg, src, w)
    c = K.Cache(plan, "cuda")
    for t in (c.ck_pool, c.cv_pool, c.dk_pool, c.dv_pool, c.rank_pool):
        t.zero_()
    g = torch.Generator().manual_seed(7)
    n = n1 + n2
    rank = torch.randint(0, 17, (B, n), generator=g).to(torch.uint8)
    ck = torch.randn(B, n, 2, 32, generator=g).to(torch.bfloat16)
    cv = torch.randn(B, n, 2, 32, generator=g).to(torch.bfloat16)
    dk = torch.randint(-127, 128, (B, n, 2, 16), generator=g).to(torch.int8)
    dv = torch.randint(-127, 128, (B, n, 2, 16), generator=g).to(torch.int8)
    sk = torch.rand(B, n, 2, generator=g).to(torch.float16)
    sv = torch.rand(B, n, 2, generator=g).to(torch.float16)
    for lo, hi in ((0, n1), (n1, n)):
        sp = torch.full((B,), lo, dtype=torch.int32).cuda()
        K.kvs_append_factorized(plan, c, 0, ck[:, lo:hi].contiguous().cuda(),
                                cv[:, lo:hi].contiguous().cuda(), dk[:, lo:hi].contiguous().cuda(),
                                dv[:, lo:hi].contiguous().cuda(), sk[:, lo:hi].contiguous().cuda(),
                                sv[:, lo:hi].contiguous().cuda(), rank[:, lo:hi].contiguous().cuda(), sp)
    torch.cuda.synchronize()
    sz = c.sizes
    P = sz.n_phys_pages
    pt = c.page_table.cpu().view(B, -1)
    ckp = c.ck_pool.cpu().view(torch.int16).view(-1, P, 2, 64 * 32)
    cvp = c.cv_pool.cpu().view(torch.int16).view(-1, P, 2, 64 * 32)
    dkp = c.dk_pool.cpu().view(torch.int8).view(-1, P, 2, 128 * 8)
    dvp = c.dv_pool.cpu().view(torch.int8).view(-1, P, 2, 128 * 8)
    meta = c.rank_pool.cpu().view(torch.int16).view(P, 64).to(torch.int32) & 0xffff
    ck16, cv16 = ck.view(torch.int16), cv.view(torch.int16)
    for b in range(B):
        goff = 0
        for pos in range(n):
            page, t = int(pt[b, pos // 64]), pos % 64
            if t == 0:
                goff = 0
            r = int(rank[b, pos])
            assert int(meta[page, t]) == r | (goff << 8), (b, pos)
            for h in range(2):
                for i in range(32):
                    assert int(ckp[0, page, h, ((i // 8) * 64 + t) * 8 + i % 8]) == int(ck16[b, pos, h, i])
                    m, j = i // 4, i % 4
                    ln = 4 * (t // 4) + j
                    off = ((m // 2) * 64 + ln) * 8 + (m % 2) * 4 + t % 4
                    assert int(cvp[0, page, h, off]) == int(cv16[b, pos, h, i])
                ng = (r + 7) // 8
                for j in range(8 * ng):
                    want_k = int(dk[b, pos, h, j]) if j < r else 0
                    want_v = int(dv[b, pos, h, j]) if j < r else 0
                    assert int(dkp[0, page, h, goff * 8 + j]) == want_k, (b, pos, h, j)
                    assert int(dvp[0, page, h, goff * 8 + j]) == want_v, (b, pos, h, j)
            goff += (r + 7) // 8


def test_factorized_append_skips_positions_out_of_range():
    """Positions below 0 or at max_ctx and beyond are skipped: sequence 0's
    chunk starts before position 0, sequence 1's runs past the context end.
    The written tokens' meta entries (rank | granule offset << 8), codes and
    scales follow the layout; the skipped slots stay untouched (zero)."""
    wl = F.with_(n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64)
    B, ctx, n = 2, 192, 70
    import attention_cross_layer_amd as K
    note(f"[factorized append range] B={B} ctx={ctx} n={n} start=(-10, {ctx - 30})")
    src, w = datagen.share_map(wl)
    cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", B, ctx,
                        kind=K.KVS_FACTORIZED, basis_rank=32, resid_rank_max=16)
    plan = K.kvs_share_plan(cfg, src, w)
    c = K.Cache(plan, "cuda")
    for t in (c.ck_pool, c.cv_pool, c.dk_pool, c.dv_pool, c.sk_pool, c.rank_pool):
        t.zero_()
    g = torch.Generator().manual_seed(11)
    rank = torch.randint(0, 17, (B, n), generator=g).to(torch.uint8)
    ck = torch.randn(B, n, 2, 32, generator=g).to(torch.bfloat16)
    cv = torch.randn(B, n, 2, 32, generator=g).to(torch.bfloat16)
    dk = torch.randint(-127, 128, (B, n, 2, 16), generator=g).to(torch.int8)
    dv = torch.randint(-127, 128, (B, n, 2, 16), generator=g).to(torch.int8)
    sk = (torch.rand(B, n, 2, generator=g) + 0.5).to(torch.float16)
    sv = (torch.rand(B, n, 2, generator=g) + 0.5).to(torch.float16)
    starts = [-10, ctx - 30]
    sp = torch.tensor(starts, dtype=torch.int32).cuda()
    K.kvs_append_factorized(plan, c, 0, ck.cuda(), cv.cuda(), dk.cuda(), dv.cuda(), sk.cuda(),
                            sv.cuda(), rank.cuda(), sp)
    torch.cuda.synchronize()
    P = c.sizes.n_phys_pages
    pt = c.page_table.cpu().view(B, -1)
    dkp = c.dk_pool.cpu().view(torch.int8).view(-1, P, 2, 128 * 8)
    skp = c.sk_pool.cpu().view(torch.int16).view(-1, P, 2, 64)
    meta = c.rank_pool.cpu().view(torch.int16).view(P, 64).to(torch.int32) & 0xffff
    sk16 = sk.view(torch.int16)
    for b in range(B):
        written = {starts[b] + i: i for i in range(n) if 0 <= starts[b] + i < ctx}
        goff = 0
        for pos in range(ctx):
            page, t = int(pt[b, pos // 64]), pos % 64
            if t == 0:
                goff = 0
            if pos not in written:
                assert int(meta[page, t]) == 0, (b, pos)
                assert all(int(skp[0, page, h, t]) == 0 for h in range(2)), (b, pos)
                continue
            i = written[pos]
            r = int(rank[b, i])
            assert int(meta[page, t]) == r | (goff << 8), (b, pos)
            for h in range(2):
                assert int(skp[0, page, h, t]) == int(sk16[b, i, h]), (b, pos, h)
                for j in range(8 * ((r + 7) // 8)):
                    want = int(dk[b, i, h, j]) if j < r else 0
                    assert int(dkp[0, page, h, goff * 8 + j]) == want, (b, pos, h, j)
            goff += (r + 7) // 8
