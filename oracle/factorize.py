"""fp64 reference for the write side of the factorized cache: the pair basis,
each layer's residual directions, and the encoder that turns a layer's K (or
V) rows into pair coefficients plus int8 residual codes with a per-token
scale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "DepthWeave-KV: Smarter KV Cache Compression by Sharing Across Layers
and Adapting Per Token", Core Mechanism (a low-rank channel basis shared by a
pair of neighbouring layers, computed without training or a calibration
set; each layer's K/V rebuilt as its basis part plus a small, low-rank,
quantized per-layer residual; a per-token reconstruction rank) and Key
Concepts (cross-layer residual factorization).  The page names none of the
numerical steps.  Readings (each also listed with the design notes):

* Basis of a pair, per KV head: the R leading right singular vectors of the
  token rows of both layers stacked (uncentred principal directions over
  every counted token of every sequence).  Row i is the i-th direction;
  each row's sign makes its largest-magnitude entry positive.
* Coefficients of token t: c = B x_t of the pair's coefficient-writing layer
  (the rows of B are orthonormal, so these are the least-squares
  coordinates), rounded to bf16 as the cache stores them.
* Residual directions of layer l: the Rmax leading right singular vectors of
  the layer's residual rows x_t - c_t B (c_t from the coefficient-writing
  layer, B as stored in bf16).
* Codes of token t with rank r: y = U (x_t - c_t B); scale s = max_{j<r} |y_j|
  / 127 rounded to fp16; d_j = round-half-even(y_j / s) clamped to
  [-127, 127] for j < r and 0 for j >= r; s = 0 and all codes 0 when r = 0 or
  the maximum is 0.

Tensor layouts: rows [B, T, Hkv, hd]; bases [Hkv, k, hd]; token counts
``lens`` [B] (tokens t < lens[b] of sequence b count).
"""
from __future__ import annotations

import numpy as np

from .attention import f64


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even; finite normal-range values (the cache's coefficients)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_fp16(x) -> np.ndarray:
    """Round float64 values to the nearest IEEE half (subnormals included),
    ties to even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def leading_directions(rows, k: int) -> np.ndarray:
    """The k leading right singular vectors of ``rows`` [N, hd] as rows of a
    [k, hd] array, largest singular value first, each row's largest-magnitude
    entry positive.  With fewer than k nonzero singular values the trailing
    rows complete an orthonormal set and are not unique."""
    rows = f64(rows)
    _, _, vt = np.linalg.svd(rows, full_matrices=True)
    out = vt[:k].copy()
    for i in range(out.shape[0]):
        j = int(np.argmax(np.abs(out[i])))
        if out[i, j] < 0:
            out[i] = -out[i]
    return out


def _counted_rows(x, lens, g):
    """Rows of KV head g over the counted tokens of every sequence, [N, hd]."""
    x = f64(x)
    return np.concatenate([x[b, :int(lens[b]), g, :] for b in range(x.shape[0])], axis=0)


def pair_basis(xa, xb, lens, rank: int) -> np.ndarray:
    """Basis of a layer pair, [Hkv, rank, hd] float64: per KV head the leading
    directions of the two layers' token rows stacked."""
    Hkv = f64(xa).shape[2]
    out = []
    for g in range(Hkv):
        rows = np.concatenate([_counted_rows(xa, lens, g), _counted_rows(xb, lens, g)], axis=0)
        out.append(leading_directions(rows, rank))
    return np.stack(out)


def coefficients(x_owner, basis) -> np.ndarray:
    """Pair coefficients of every token, rounded to bf16: [B, T, Hkv, R]."""
    return round_bf16(np.einsum("btgd,gid->btgi", f64(x_owner), f64(basis)))


def residual_rows(x, x_owner, basis) -> np.ndarray:
    """x - c B with c the stored (bf16) coefficients from the coefficient-
    writing layer's rows: [B, T, Hkv, hd]."""
    c = coefficients(x_owner, basis)
    return f64(x) - np.einsum("btgi,gid->btgd", c, f64(basis))


def residual_basis(x, x_owner, basis, lens, rmax: int) -> np.ndarray:
    """Residual directions of a layer, [Hkv, rmax, hd] float64."""
    e = residual_rows(x, x_owner, basis)
    return np.stack([leading_directions(_counted_rows(e, lens, g), rmax)
                     for g in range(e.shape[2])])


def encode(x, x_owner, basis, ubasis, rank):
    """Encode a layer's rows.

    x, x_owner [B, T, Hkv, hd]; basis [Hkv, R, hd] and ubasis [Hkv, Rmax, hd]
    as stored (bf16 values); rank [B, T].
    Returns (c [B,T,Hkv,R] bf16 values, y [B,T,Hkv,Rmax] the unquantized
    residual coordinates, s [B,T,Hkv] fp16 values, d [B,T,Hkv,Rmax] int
    codes), all float64 except d (int64).
    """
    c = coefficients(x_owner, basis)
    e = f64(x) - np.einsum("btgi,gid->btgd", c, f64(basis))
    y = np.einsum("btgd,gjd->btgj", e, f64(ubasis))
    rmax = y.shape[-1]
    r = f64(rank)
    keep = np.arange(rmax)[None, None, None, :] < r[:, :, None, None]
    amax = np.max(np.where(keep, np.abs(y), 0.0), axis=-1)
    s = round_fp16(amax / 127.0)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(y / safe[..., None]), -127, 127)
    d = np.where(keep & (s[..., None] > 0), q, 0.0).astype(np.int64)
    return c, y, s, d
