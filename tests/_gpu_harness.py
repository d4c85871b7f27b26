"""Shared set-up for the GPU parity tests: build a plan and a cache through the
library, fill owner slots with seeded K/V via kvs_append, and compare
library outputs with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from oracle import plan as P

TOL_ABS = 1e-2     # max-abs error bound for bf16 inputs with fp32 accumulation
TOL_REL = 5e-3     # relative L2 error bound
TOL_F32 = 2e-5     # fp32 inputs: accumulation-order rounding only


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got: torch.Tensor, ref: np.ndarray):
    g = got.detach().to("cpu", torch.float64).numpy()
    d = g - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d)) / den if den > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(got, ref, dtype="bf16", what=""):
    max_abs, rel = errors(got, ref)
    if dtype == "f32":
        assert max_abs <= TOL_F32, f"{what}: max_abs {max_abs:.3e}"
    else:
        assert max_abs <= TOL_ABS and rel <= TOL_REL, f"{what}: max_abs {max_abs:.3e} rel {rel:.3e}"
    return max_abs, rel


class Dense:
    """A dense shared cache for a workload, populated through kvs_append."""

    def __init__(self, wl: datagen.Workload, batch: int, ctx: int, lens, page_perm=None,
                 kv_device="cpu", nan_fill=True, append_lens=None):
        self.wl = wl
        self.batch, self.ctx = batch, ctx
        self.src, self.w = datagen.share_map(wl)
        cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.dtype,
                            batch, ctx)
        self.plan = K.kvs_share_plan(cfg, self.src, self.w)
        self.cache = K.Cache(self.plan, "cuda", page_perm=page_perm)
        if nan_fill == "zero":
            self.cache.k_pool.zero_()
            self.cache.v_pool.zero_()
        elif nan_fill:   # unwritten cache memory holds NaN patterns
            self.cache.k_pool.fill_(0xFF)
            self.cache.v_pool.fill_(0xFF)
        self.owners = datagen.owner_layers(self.src)
        self.k, self.v = {}, {}
        self.lens = torch.tensor(lens, dtype=torch.int32)
        self.seq_len = self.lens.cuda()
        app = self.lens if append_lens is None else torch.tensor(append_lens, dtype=torch.int32)
        for l in self.owners:
            k, v = datagen.owner_kv(wl, l, device=kv_device, batch=batch, ctx=ctx)
            self.k[l], self.v[l] = k.cpu(), v.cpu()
            kd, vd = k.cuda(), v.cuda()
            # one call per sequence, appending exactly its own tokens; the other
            # sequences get a start position past capacity and are skipped
            for b in range(batch):
                n = int(app[b])
                if n == 0:
                    continue
                sp = torch.full((batch,), ctx, dtype=torch.int32)
                sp[b] = 0
                K.kvs_append(self.plan, self.cache, l, kd[:, :n].contiguous(),
                             vd[:, :n].contiguous(), sp.cuda())
        torch.cuda.synchronize()

    def q(self, layer):
        return datagen.decode_q(self.wl, layer, batch=self.batch)

    def decode(self, layer, q=None, n_splits=0, out_dtype=torch.float32):
        q = self.q(layer) if q is None else q
        return K.kvs_attn_decode(self.plan, self.cache, layer, q.cuda(), self.seq_len,
                                 int(self.lens.max()), n_splits=n_splits, out_dtype=out_dtype)

    def oracle_decode(self, layer, q=None):
        q = self.q(layer) if q is None else q
        return A.layer_decode(self.src.tolist(), self.w.tolist(), layer, self.k, self.v, q,
                              self.lens.tolist())


class Factorized:
    """A factorized shared cache (pair basis + per-layer int8 residual),
    populated through kvs_append_factorized; bases copied into the cache's
    basis buffers."""

    def __init__(self, wl: datagen.Workload, batch: int, ctx: int, lens, junk=True,
                 dev_gen="cpu", rank_override=None, scale_zero=False):
        self.wl, self.batch, self.ctx = wl, batch, ctx
        self.src, self.w = datagen.share_map(wl)
        cfg = K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16", batch,
                            ctx, kind=K.KVS_FACTORIZED, basis_rank=wl.basis_rank,
                            resid_rank_max=wl.resid_rank_max)
        self.plan = K.kvs_share_plan(cfg, self.src, self.w)
        self.cache = c = K.Cache(self.plan, "cuda")
        for t in (c.ck_pool, c.cv_pool, c.sk_pool, c.sv_pool, c.rank_pool, c.dk_pool, c.dv_pool):
            t.fill_(0xFF)           # unwritten memory: NaN patterns, rank 255, codes -1
        self.lens = torch.tensor(lens, dtype=torch.int32)
        self.seq_len = self.lens.cuda()
        Hkv, R, Rm, hd = wl.n_kv_heads, wl.basis_rank, wl.resid_rank_max, wl.head_dim
        n_slots = c.sizes.n_slots
        self.rank = (datagen.token_ranks(wl, device=dev_gen, batch=batch, ctx=ctx)
                     if rank_override is None else rank_override).cpu()
        bk_all = c.basis_k.view(torch.bfloat16).view(n_slots, Hkv, R, hd)
        bv_all = c.basis_v.view(torch.bfloat16).view(n_slots, Hkv, R, hd)
        uk_all = c.ubasis_k.view(torch.bfloat16).view(wl.n_layers, Hkv, Rm, hd)
        uv_all = c.ubasis_v.view(torch.bfloat16).view(wl.n_layers, Hkv, Rm, hd)
        self.coef, self.basis, self.resid, self.ubasis = {}, {}, {}, {}
        owners = datagen.owner_layers(self.src)
        for l in range(wl.n_layers):
            pair = int(self.src[l, 0])
            if l in owners:
                ck, cv = datagen.pair_coeffs(wl, pair // 2, device=dev_gen, batch=batch, ctx=ctx)
                bk, bv = datagen.pair_basis(wl, pair // 2, device=dev_gen)
                slot = owners.index(l)
                bk_all[slot].copy_(bk)
                bv_all[slot].copy_(bv)
                self.coef[l] = (ck.cpu(), cv.cpu())
                self.basis[l] = (bk.cpu(), bv.cpu())
            uk, uv = datagen.layer_residual_basis(wl, l, device=dev_gen)
            uk_all[l].copy_(uk)
            uv_all[l].copy_(uv)
            dk, dv, sk, sv = datagen.layer_residual(wl, l, self.rank.to(dev_gen), device=dev_gen,
                                                    junk_beyond_rank=junk)
            if scale_zero:
                sk, sv = torch.zeros_like(sk), torch.zeros_like(sv)
            self.resid[l] = (dk.cpu(), dv.cpu(), sk.cpu(), sv.cpu())
            self.ubasis[l] = (uk.cpu(), uv.cpu())
            for b in range(batch):
                n = int(self.lens[b])
                if n == 0:
                    continue
                sp = torch.full((batch,), ctx, dtype=torch.int32)
                sp[b] = 0
                coefs = self.coef.get(l)
                K.kvs_append_factorized(
                    self.plan, self.cache, l,
                    None if coefs is None else coefs[0][:, :n].contiguous().cuda(),
                    None if coefs is None else coefs[1][:, :n].contiguous().cuda(),
                    dk[:, :n].contiguous().cuda(), dv[:, :n].contiguous().cuda(),
                    sk[:, :n].contiguous().cuda(), sv[:, :n].contiguous().cuda(),
                    self.rank[:, :n].contiguous().cuda(), sp.cuda())
        torch.cuda.synchronize()

    def q(self, layer):
        return datagen.decode_q(self.wl, layer, batch=self.batch)

    def decode(self, layer, q=None, n_splits=0, out_dtype=torch.float32):
        q = self.q(layer) if q is None else q
        return K.kvs_attn_decode(self.plan, self.cache, layer, q.cuda(), self.seq_len,
                                 int(self.lens.max()), n_splits=n_splits, out_dtype=out_dtype)

    def kv(self, layer, b0=0, b1=None):
        """Oracle reconstruction of layer's K, V (float64) for sequences b0..b1."""
        pair = int(self.src[layer, 0])
        ck, cv = (x[b0:b1] for x in self.coef[pair])
        bk, bv = self.basis[pair]
        dk, dv, sk, sv = (x[b0:b1] for x in self.resid[layer])
        uk, uv = self.ubasis[layer]
        r = self.rank[b0:b1]
        return A.factorized_kv(ck, bk, sk, dk, uk, r), A.factorized_kv(cv, bv, sv, dv, uv, r)

    def oracle_decode(self, layer, q=None):
        q = self.q(layer) if q is None else q
        k, v = self.kv(layer)
        return A.attend_decode(q, k, v, self.lens.tolist(),
                               exclude_current=P.excludes_current(self.src.tolist(), self.w.tolist(), layer))

    def prefill(self, layer, q, causal=True, out_dtype=torch.float32):
        got = K.kvs_attn_prefill_chunk(self.plan, self.cache, layer, q.cuda(), self.seq_len,
                                       causal=causal, out_dtype=out_dtype)
        torch.cuda.synchronize()
        return got

    def oracle_prefill(self, layer, q, causal=True):
        k, v = self.kv(layer)
        return A.attend_prefill(q, k, v, self.lens.tolist(), causal=causal,
                                exclude_current=P.excludes_current(self.src.tolist(), self.w.tolist(), layer))


def unpack_factorized(cache, layer, slot, B, n, Hkv, start=0):
    """Read back the factorized entries of positions start..start+n-1 of every
    sequence (page table of ``cache``) into dense host arrays, following the
    documented pool layout: coefficients of ``slot`` (cK, cV: [B,n,Hkv,32]
    bf16 as float64), codes of ``layer`` (dK, dV: [B,n,Hkv,16] int), scales
    (sK, sV: [B,n,Hkv] float64) and ranks [B,n]."""
    sz = cache.sizes
    P_ = sz.n_phys_pages
    pt = cache.page_table.cpu()
    ckp = cache.ck_pool.cpu().view(torch.bfloat16).view(-1, P_, Hkv, 64 * 32).double().numpy()
    cvp = cache.cv_pool.cpu().view(torch.bfloat16).view(-1, P_, Hkv, 64 * 32).double().numpy()
    dkp = cache.dk_pool.cpu().view(torch.int8).view(-1, P_, Hkv, 128 * 8).numpy().astype(np.int64)
    dvp = cache.dv_pool.cpu().view(torch.int8).view(-1, P_, Hkv, 128 * 8).numpy().astype(np.int64)
    skp = cache.sk_pool.cpu().view(torch.float16).view(-1, P_, Hkv, 64).double().numpy()
    svp = cache.sv_pool.cpu().view(torch.float16).view(-1, P_, Hkv, 64).double().numpy()
    meta = cache.rank_pool.cpu().view(torch.int16).view(P_, 64).numpy().astype(np.int64) & 0xffff
    ck = np.zeros((B, n, Hkv, 32)); cv = np.zeros((B, n, Hkv, 32))
    dk = np.zeros((B, n, Hkv, 16), dtype=np.int64); dv = np.zeros((B, n, Hkv, 16), dtype=np.int64)
    sk = np.zeros((B, n, Hkv)); sv = np.zeros((B, n, Hkv))
    rank = np.zeros((B, n), dtype=np.int64)
    i_idx = np.arange(32)
    m = i_idx // 4
    for b in range(B):
        for i in range(n):
            pos = start + i
            page, t = int(pt[b, pos // 64]), pos % 64
            r, o = int(meta[page, t]) & 0xff, int(meta[page, t]) >> 8
            rank[b, i] = r
            cvo = ((m // 2) * 64 + 4 * (t // 4) + i_idx % 4) * 8 + (m % 2) * 4 + t % 4
            cko = ((i_idx // 8) * 64 + t) * 8 + i_idx % 8
            for h in range(Hkv):
                ck[b, i, h] = ckp[slot, page, h, cko]
                cv[b, i, h] = cvp[slot, page, h, cvo]
                nb = 8 * ((r + 7) // 8)
                dk[b, i, h, :nb] = dkp[layer, page, h, o * 8:o * 8 + nb]
                dv[b, i, h, :nb] = dvp[layer, page, h, o * 8:o * 8 + nb]
                sk[b, i, h] = skp[layer, page, h, t]
                sv[b, i, h] = svp[layer, page, h, t]
    return ck, cv, dk, dv, sk, sv, rank
