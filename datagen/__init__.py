"""Seeded synthetic inputs for the shared-KV attention path.

This module is the one piece that both the CPU oracle side (tests, the
oracle's timing leg) and the HIP side (tests, the benchmark) consume.  It
draws random tensors and builds the layer->source tables of each workload;
it performs none of the method's arithmetic (no attention, no mixing of
sources, no reconstruction of factorized keys/values).

Every tensor comes from its own ``torch.Generator`` seeded from
``(workload seed, tensor tag, index)``, so any tensor can be regenerated on
its own, on the CPU or on a GPU.  The two devices produce different streams;
a consumer that needs the same values on both sides generates once and
copies.

Workloads (sizes from the task's stated configurations; the value
distributions are the readings recorded in the design notes):

* ``tiny_cla2``      4 layers, map [0,0,2,2] (CLA2), batch 1, 4 q / 2 KV heads,
                     head_dim 64, context 128, fp32.
* ``tinyllama_cla2`` 22 layers, CLA2 (11 cached layers), 32 q / 4 KV heads,
                     head_dim 64, bf16, batch 64, context 2048 (the 1.1B shape
                     whose generation throughput the cross-layer-sharing study
                     plots in its Figure 2: prompt 5 + generation 2043).
* ``depthgraft``     24 layers, layers 0-15 own KV, layer l >= 16 mixes layers
                     l-8 and l-16 with weights a_l and 1-a_l, a_l ~ U(0,1);
                     32 q / 8 KV heads, head_dim 128, bf16, batch 8 decode at
                     context 8192, plus a 4096-token causal prefill chunk.
* ``cla2_64k``       32 layers, CLA2, 32 q / 8 KV heads, head_dim 128, bf16,
                     batch 4, context 65536; 1% of keys per (layer, batch,
                     KV head) scaled by 4 (peaky attention).
* ``factorized_64k`` 32 layers in 16 pairs; per KV head
                     K/V[t] = c[t] B_pair + s[t] d_l[t] U_l, basis rank 32,
                     int8 residual rank r_t in {0, 8, 16} (10% rank 16),
                     fp16 scale; 32 q / 8 KV heads, head_dim 128, batch 2,
                     context 65536.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import torch

PAGE = 64  # tokens per cache page / key block

TAG_K, TAG_V, TAG_Q, TAG_QP, TAG_PEAK, TAG_MIX = 1, 2, 3, 4, 5, 6
TAG_CK, TAG_CV, TAG_BK, TAG_BV, TAG_DK, TAG_DV = 11, 12, 13, 14, 15, 16
TAG_SK, TAG_SV, TAG_UK, TAG_UV, TAG_RANK = 17, 18, 19, 20, 21
TAG_PAIR_DIR, TAG_PAIR_LATENT, TAG_LAYER_DIR, TAG_LAYER_LATENT, TAG_NOISE = 22, 23, 24, 25, 26


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16": cache, q and prefill q dtype
    batch: int
    ctx: int                   # keys visible to the decode query (incl. itself)
    seed: int
    kind: str = "dense"        # "dense" or "factorized"
    share: str = "cla2"        # "cla2", "cla2_top", "mid3", "depthgraft", "identity", "pairs", "pairs_top"
    peaky_frac: float = 0.0    # fraction of keys whose vector is scaled by 4
    prefill_n: int = 0         # prefill chunk length (0: none)
    prefill_batch: int = 0
    basis_rank: int = 0
    resid_rank_max: int = 0
    rank16_frac: float = 0.0
    dg_stride: int = 8         # depthgraft: layers >= 2*stride mix l-stride, l-2*stride

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_cla2": Workload("tiny_cla2", 4, 4, 2, 64, "f32", 1, 128, 0x5EED0 + 1),
    "tinyllama_cla2": Workload("tinyllama_cla2", 22, 32, 4, 64, "bf16", 64, 2048,
                               0x5EED0 + 2),
    "depthgraft": Workload("depthgraft", 24, 32, 8, 128, "bf16", 8, 8192, 0x5EED0 + 3,
                           share="depthgraft", prefill_n=4096, prefill_batch=1),
    "cla2_64k": Workload("cla2_64k", 32, 32, 8, 128, "bf16", 4, 65536, 0x5EED0 + 4,
                         peaky_frac=0.01),
    "factorized_64k": Workload("factorized_64k", 32, 32, 8, 128, "bf16", 2, 65536,
                               0x5EED0 + 5, kind="factorized", share="pairs",
                               basis_rank=32, resid_rank_max=16, rank16_frac=0.1),
    # the 1.1B shape with each adjacent pair served by its upper layer (a top
    # configuration of the systematic cross-layer KV sharing study)
    "tinyllama_cla2_top": Workload("tinyllama_cla2_top", 22, 32, 4, 64, "bf16", 64, 2048,
                                   0x5EED0 + 6, share="cla2_top"),
}


def _gen(wl: Workload, tag: int, index: int, device) -> torch.Generator:
    seed = (wl.seed * 1_000_003 + tag * 10_007 + index) % (2 ** 62)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# ----------------------------------------------------------------------------
# layer -> source tables
# ----------------------------------------------------------------------------

def share_map(wl: Workload, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Return (src [L,2] int32, w [L,2] float32) for the workload.

    Row l lists the layers whose cached K/V layer l reads and their weights;
    an unused second entry is (-1, 0).  A layer that computes and caches its
    own K/V has row (l, 1.0), (-1, 0).
    """
    L = wl.n_layers
    src = torch.full((L, 2), -1, dtype=torch.int32)
    w = torch.zeros((L, 2), dtype=torch.float32)
    if wl.share in ("cla2", "pairs"):
        for l in range(L):
            src[l, 0] = 2 * (l // 2)
            w[l, 0] = 1.0
    elif wl.share in ("cla2_top", "pairs_top"):
        # adjacent pairs whose upper layer holds the K/V (a top configuration)
        for l in range(L):
            src[l, 0] = min(2 * (l // 2) + 1, L - 1)
            w[l, 0] = 1.0
    elif wl.share == "mid3":
        # groups of three layers served by the middle one (a middle configuration)
        for l in range(L):
            src[l, 0] = min(3 * (l // 3) + 1, L - 1)
            w[l, 0] = 1.0
    elif wl.share == "identity":
        for l in range(L):
            src[l, 0] = l
            w[l, 0] = 1.0
    elif wl.share == "depthgraft":
        a = torch.rand(L, generator=_gen(wl, TAG_MIX, 0, "cpu"), dtype=torch.float32)
        stride = wl.dg_stride
        n_own = 2 * stride
        for l in range(L):
            if l < n_own:
                src[l, 0] = l
                w[l, 0] = 1.0
            else:
                src[l, 0] = l - stride
                src[l, 1] = l - 2 * stride
                w[l, 0] = a[l]
                # the second weight is part of the input table: 1 - a in fp32
                w[l, 1] = torch.tensor(1.0, dtype=torch.float32) - a[l]
    else:
        raise ValueError(wl.share)
    return src, w


def owner_layers(src: torch.Tensor) -> list:
    return [l for l in range(src.shape[0]) if int(src[l, 0]) == l and int(src[l, 1]) < 0]


# ----------------------------------------------------------------------------
# dense K/V, queries
# ----------------------------------------------------------------------------

def owner_kv(wl: Workload, layer: int, device="cpu", batch: Optional[int] = None,
             ctx: Optional[int] = None):
    """K, V of an owner layer, layout [B, T, Hkv, hd] in the workload dtype.

    Values ~ N(0,1) drawn in fp32 and rounded to the storage dtype.  With
    ``peaky_frac`` > 0, exactly round(frac * T) positions per (batch, KV head),
    chosen by a seeded permutation, have their key vector multiplied by 4.
    """
    B = wl.batch if batch is None else batch
    T = wl.ctx if ctx is None else ctx
    shape = (B, T, wl.n_kv_heads, wl.head_dim)
    k = torch.randn(shape, generator=_gen(wl, TAG_K, layer, device), device=device,
                    dtype=torch.float32)
    v = torch.randn(shape, generator=_gen(wl, TAG_V, layer, device), device=device,
                    dtype=torch.float32)
    if wl.peaky_frac > 0.0:
        n_peak = int(round(wl.peaky_frac * T))
        g = _gen(wl, TAG_PEAK, layer, device)
        for b in range(B):
            for h in range(wl.n_kv_heads):
                pos = torch.randperm(T, generator=g, device=device)[:n_peak]
                k[b, pos, h, :] *= 4.0
    return k.to(wl.torch_dtype), v.to(wl.torch_dtype)


def decode_q(wl: Workload, layer: int, device="cpu", batch: Optional[int] = None):
    """Decode query of a layer, [B, Hq, hd] in the workload dtype, ~N(0,1)."""
    B = wl.batch if batch is None else batch
    q = torch.randn((B, wl.n_q_heads, wl.head_dim), generator=_gen(wl, TAG_Q, layer, device),
                    device=device, dtype=torch.float32)
    return q.to(wl.torch_dtype)


def prefill_q(wl: Workload, layer: int, n: int, device="cpu", batch: Optional[int] = None):
    """Prefill-chunk queries of a layer, [B, n, Hq, hd], ~N(0,1)."""
    B = wl.batch if batch is None else batch
    q = torch.randn((B, n, wl.n_q_heads, wl.head_dim),
                    generator=_gen(wl, TAG_QP, layer, device), device=device,
                    dtype=torch.float32)
    return q.to(wl.torch_dtype)


# ----------------------------------------------------------------------------
# factorized cache inputs
# ----------------------------------------------------------------------------

def token_ranks(wl: Workload, device="cpu", batch: Optional[int] = None,
                ctx: Optional[int] = None, ranks: Sequence[int] = (0, 8, 16)):
    """Residual rank per (batch, token), uint8 [B, T].

    Exactly round(rank16_frac * T) tokens per sequence get the top rank; the
    rest are split evenly between the two lower ranks (the odd one goes to
    the lowest); positions come from a seeded permutation.
    """
    B = wl.batch if batch is None else batch
    T = wl.ctx if ctx is None else ctx
    lo, mid, hi = ranks
    n_hi = int(round(wl.rank16_frac * T))
    n_mid = (T - n_hi) // 2
    out = torch.empty((B, T), dtype=torch.uint8, device=device)
    g = _gen(wl, TAG_RANK, 0, device)
    for b in range(B):
        perm = torch.randperm(T, generator=g, device=device)
        r = torch.full((T,), lo, dtype=torch.uint8, device=device)
        r[perm[:n_hi]] = hi
        r[perm[n_hi:n_hi + n_mid]] = mid
        out[b] = r
    return out


def pair_coeffs(wl: Workload, pair: int, device="cpu", batch=None, ctx=None):
    """Pair-shared coefficients cK, cV: [B, T, Hkv, R] bf16, ~N(0,1)."""
    B = wl.batch if batch is None else batch
    T = wl.ctx if ctx is None else ctx
    shape = (B, T, wl.n_kv_heads, wl.basis_rank)
    ck = torch.randn(shape, generator=_gen(wl, TAG_CK, pair, device), device=device)
    cv = torch.randn(shape, generator=_gen(wl, TAG_CV, pair, device), device=device)
    return ck.to(torch.bfloat16), cv.to(torch.bfloat16)


def pair_basis(wl: Workload, pair: int, device="cpu"):
    """Pair basis BK, BV: [Hkv, R, hd] bf16, ~N(0,1)/sqrt(R)."""
    shape = (wl.n_kv_heads, wl.basis_rank, wl.head_dim)
    f = 1.0 / math.sqrt(wl.basis_rank)
    bk = torch.randn(shape, generator=_gen(wl, TAG_BK, pair, device), device=device) * f
    bv = torch.randn(shape, generator=_gen(wl, TAG_BV, pair, device), device=device) * f
    return bk.to(torch.bfloat16), bv.to(torch.bfloat16)


def layer_residual_basis(wl: Workload, layer: int, device="cpu"):
    """Per-layer residual directions UK, UV: [Hkv, Rmax, hd] bf16, ~N(0,1)/4."""
    shape = (wl.n_kv_heads, wl.resid_rank_max, wl.head_dim)
    uk = torch.randn(shape, generator=_gen(wl, TAG_UK, layer, device), device=device) * 0.25
    uv = torch.randn(shape, generator=_gen(wl, TAG_UV, layer, device), device=device) * 0.25
    return uk.to(torch.bfloat16), uv.to(torch.bfloat16)


def layer_residual(wl: Workload, layer: int, rank: torch.Tensor, device="cpu",
                   junk_beyond_rank: bool = False):
    """Per-layer int8 residual codes and fp16 scales.

    Returns dK, dV int8 [B, T, Hkv, Rmax] (uniform integers in [-127, 127];
    entries at index >= r_t are zero, or random junk when
    ``junk_beyond_rank`` so a consumer that ignores r_t is caught) and
    sK, sV fp16 [B, T, Hkv] = U(0.5, 1.5) * 0.5 / 127.
    """
    B, T = rank.shape
    shape = (B, T, wl.n_kv_heads, wl.resid_rank_max)
    gk = _gen(wl, TAG_DK, layer, device)
    gv = _gen(wl, TAG_DV, layer, device)
    dk = torch.randint(-127, 128, shape, generator=gk, device=device, dtype=torch.int32)
    dv = torch.randint(-127, 128, shape, generator=gv, device=device, dtype=torch.int32)
    if not junk_beyond_rank:
        j = torch.arange(wl.resid_rank_max, device=device).view(1, 1, 1, -1)
        keep = j < rank.to(torch.int32).view(B, T, 1, 1)
        dk = torch.where(keep, dk, torch.zeros_like(dk))
        dv = torch.where(keep, dv, torch.zeros_like(dv))
    sshape = (B, T, wl.n_kv_heads)
    sk = torch.rand(sshape, generator=_gen(wl, TAG_SK, layer, device), device=device)
    sv = torch.rand(sshape, generator=_gen(wl, TAG_SV, layer, device), device=device)
    sk = ((sk + 0.5) * (0.5 / 127.0)).to(torch.float16)
    sv = ((sv + 0.5) * (0.5 / 127.0)).to(torch.float16)
    return dk.to(torch.int8), dv.to(torch.int8), sk, sv


def _orthonormal_rows(k: int, hd: int, g: torch.Generator, device) -> torch.Tensor:
    """k random orthonormal rows [k, hd] (QR of a Gaussian matrix)."""
    m = torch.randn((hd, k), generator=g, device=device, dtype=torch.float32)
    q, r = torch.linalg.qr(m.cpu().double())
    q = q * torch.sign(torch.diagonal(r))[None, :]
    return q.T.to(torch.float32).to(device)


def correlated_pair_rows(wl: Workload, pair: int, which: str, device="cpu",
                         batch: Optional[int] = None, ctx: Optional[int] = None):
    """Full K (which="k") or V ("v") rows of the two layers of a pair whose
    states are strongly correlated, the situation the factorized cache
    targets: [B, T, Hkv, hd] bf16 each, (rows of the lower layer, rows of the
    upper layer).

    Per KV head: a shared latent z_t in R^R with per-direction scales drawn
    from U(1, 2) on R random orthonormal directions; the upper layer's latent
    is z_t + 0.1 * N(0, 1) (per direction, scaled alike); each layer adds
    Rmax layer-specific random directions with N(0, 1) * U(0.3, 0.45)
    weights, and i.i.d. N(0, 0.02^2) noise on every channel.  With the
    workload's R = 32, Rmax = 16 and hd = 128 this leaves a clear gap after
    the R-th principal direction of the stacked rows and after the Rmax-th
    of each layer's residual.
    """
    B = wl.batch if batch is None else batch
    T = wl.ctx if ctx is None else ctx
    Hkv, hd, R, Rm = wl.n_kv_heads, wl.head_dim, wl.basis_rank, wl.resid_rank_max
    tw = 0 if which == "k" else 1
    idx = 2 * pair + tw
    gd = _gen(wl, TAG_PAIR_DIR, idx, "cpu")
    shared = torch.stack([_orthonormal_rows(R, hd, gd, "cpu") for _ in range(Hkv)]).to(device)
    sig = (1.0 + torch.rand((Hkv, R), generator=gd)).to(device)
    z = torch.randn((B, T, Hkv, R), generator=_gen(wl, TAG_PAIR_LATENT, idx, device),
                    device=device) * sig
    out = []
    for j in range(2):
        lj = 4 * pair + 2 * j + tw
        gl = _gen(wl, TAG_LAYER_DIR, lj, "cpu")
        own = torch.stack([_orthonormal_rows(Rm, hd, gl, "cpu") for _ in range(Hkv)]).to(device)
        tau = (0.3 + 0.15 * torch.rand((Hkv, Rm), generator=gl)).to(device)
        gz = _gen(wl, TAG_LAYER_LATENT, lj, device)
        zj = z if j == 0 else z + 0.1 * torch.randn(z.shape, generator=gz, device=device) * sig
        w = torch.randn((B, T, Hkv, Rm), generator=gz, device=device) * tau
        noise = 0.02 * torch.randn((B, T, Hkv, hd), generator=_gen(wl, TAG_NOISE, lj, device),
                                   device=device)
        x = (torch.einsum("btgi,gid->btgd", zj, shared) + torch.einsum("btgj,gjd->btgd", w, own)
             + noise)
        out.append(x.to(torch.bfloat16).contiguous())
    return out[0], out[1]


def seq_lens(batch: int, ctx: int, ragged: bool = False, seed: int = 0, min_len: int = 1):
    """Per-sequence key counts [B] int32: all ``ctx``, or seeded ragged in
    [min_len, ctx] with the first sequence at the full ``ctx``."""
    if not ragged:
        return torch.full((batch,), ctx, dtype=torch.int32)
    g = torch.Generator().manual_seed(seed)
    s = torch.randint(min_len, ctx + 1, (batch,), generator=g, dtype=torch.int32)
    s[0] = ctx
    return s
