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
