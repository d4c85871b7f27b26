"""fp64 reference attention over a cross-layer K/V sharing map.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources for what is computed:

* Attention with a K/V cache, where several query heads share one K/V head
  (GQA / MQA): "Reducing Transformer Key-Value Cache Size with Cross-Layer
  Attention" (CLA page), Abstract and Glossary entries for the KV cache, MQA
  and GQA.  The pages never print the formula; the plain reading is
  softmax(q K^T / sqrt(hd)) V per query head, query head h using K/V head
  floor(h / G) with G = Hq / Hkv (consecutive grouping).
* Reuse across layers: the CLA page, Methodology ("some layers compute new
  KV, the others reuse it") -- a reusing layer attends over the cached K/V of
  its source layer exactly as that layer would.
* Two-source mixing: "DepthGraft: Structural Regularization through
  Hierarchical Cross-Layer KV Reconstruction", Abstract (deep-layer KV
  reconstructed from stride-aligned shallow/middle source pairs).  Reading:
  the effective K (and V) of layer l is w1 * K_{s1} + w2 * K_{s2} with the
  weights of the layer's map row.
* Factorized cache: "DepthWeave-KV: Smarter KV Cache Compression by Sharing
  Across Layers and Adapting Per Token", Core Mechanism and Framework Shift
  (a channel basis shared by a layer pair plus a per-layer low-rank quantized
  residual; a per-token rank).  Reading: K_l[t] = c[t] B_pair
  + s_l[t] * sum_{j < r_t} d_l[t, j] U_l[j], the same form for V.

Tensor layouts (all logical, unpaged):
  owner K/V        [B, T, Hkv, hd]
  decode q / out   [B, Hq, hd]
  prefill q / out  [B, n, Hq, hd]
All inputs are converted to float64 exactly (bf16, fp16, fp32 and int8 values
are representable in float64).
"""
from __future__ import annotations

import numpy as np


def f64(x) -> np.ndarray:
    """Exact float64 copy of a torch tensor or array (bf16/fp16/int8 included)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def effective_kv(src_row, w_row, owner_k: dict, owner_v: dict):
    """Effective K, V of one layer: sum over the row's sources of w * K_src.

    ``src_row``/``w_row``: the layer's map row (source layers, -1 = unused;
    weights as stored fp32 values).  ``owner_k``/``owner_v`` map a source
    layer to its cached [B, T, Hkv, hd] tensor.  A single-source row with
    weight 1 returns the source tensors unchanged (CLA reuse); two sources
    give the DepthGraft-style mix.
    """
    k = None
    v = None
    for s, w in zip(src_row, w_row):
        s = int(s)
        if s < 0:
            continue
        wk = np.float64(np.float32(w)) * f64(owner_k[s])
        wv = np.float64(np.float32(w)) * f64(owner_v[s])
        k = wk if k is None else k + wk
        v = wv if v is None else v + wv
    if k is None:
        raise ValueError("map row has no source")
    return k, v


def attend_decode(q, k, v, seq_len, scale=None, exclude_current=False):
    """One query per (sequence, head) over keys 0..seq_len[b]-1.

    q [B, Hq, hd]; k, v [B, T, Hkv, hd]; returns float64 [B, Hq, hd].
    out[b, h] = sum_t softmax_t(scale * q[b,h] . k[b,t,g]) v[b,t,g],
    g = h // (Hq / Hkv), scale = 1/sqrt(hd) unless given.  With
    ``exclude_current`` the query (at position seq_len[b]-1) sees keys
    0..seq_len[b]-2 only (diagonal masking); no key at all gives zeros.
    """
    q = f64(q)
    k = f64(k)
    v = f64(v)
    B, Hq, hd = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.zeros((B, Hq, hd), dtype=np.float64)
    for b in range(B):
        T = int(seq_len[b]) - (1 if exclude_current else 0)
        if T <= 0:
            continue
        for h in range(Hq):
            g = h // G
            z = scale * (k[b, :T, g, :] @ q[b, h])
            z = z - z.max()
            e = np.exp(z)
            out[b, h] = (e @ v[b, :T, g, :]) / e.sum()
    return out


def attend_prefill(q, k, v, seq_len, causal=True, scale=None, exclude_current=False):
    """A chunk of n queries per sequence, the last n positions of the sequence.

    q [B, n, Hq, hd]; k, v [B, T, Hkv, hd] hold keys 0..seq_len[b]-1 (the chunk's
    own keys included).  Query i sits at absolute position
    P_i = seq_len[b] - n + i; with ``causal`` it sees keys 0..P_i (inclusive
    diagonal), or keys 0..P_i - 1 with ``exclude_current`` (diagonal masking),
    otherwise keys 0..seq_len[b]-1.  A query that sees no key gets zeros.
    Returns float64 [B, n, Hq, hd].
    """
    q = f64(q)
    k = f64(k)
    v = f64(v)
    B, n, Hq, hd = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.zeros((B, n, Hq, hd), dtype=np.float64)
    for b in range(B):
        T = int(seq_len[b])
        for h in range(Hq):
            g = h // G
            z = scale * (q[b, :, h, :] @ k[b, :T, g, :].T)          # [n, T]
            if causal:
                pos = T - n + np.arange(n)
                last = pos - (1 if exclude_current else 0)
                visible = np.arange(T)[None, :] <= last[:, None]
                z = np.where(visible, z, -np.inf)
            for i in range(n):
                if not np.isfinite(z[i]).any():
                    continue                      # no visible key: zeros
                zi = z[i] - z[i].max()
                e = np.exp(zi)
                out[b, i, h, :] = (e @ v[b, :T, g, :]) / e.sum()
    return out


def factorized_kv(c, basis, scale, d, u, rank):
    """Reconstruct one layer's K (or V) from the factorized cache.

    c     [B, T, Hkv, R]     coefficients shared by the layer pair
    basis [Hkv, R, hd]       the pair's channel basis
    scale [B, T, Hkv]        per-token residual scale of this layer
    d     [B, T, Hkv, Rmax]  int8 residual codes of this layer
    u     [Hkv, Rmax, hd]    this layer's residual directions
    rank  [B, T]             residual rank r_t; only codes j < r_t count
    Returns float64 [B, T, Hkv, hd]:
      K[b,t,g] = c[b,t,g] @ basis[g] + scale[b,t,g] * (d[b,t,g,:r] @ u[g,:r]).
    """
    c = f64(c)
    basis = f64(basis)
    scale = f64(scale)
    d = f64(d)
    u = f64(u)
    r = f64(rank)
    rmax = d.shape[-1]
    used = (np.arange(rmax)[None, None, :] < r[:, :, None]).astype(np.float64)  # [B,T,Rmax]
    d_used = d * used[:, :, None, :]
    base = np.einsum("btgi,gid->btgd", c, basis)
    resid = np.einsum("btgj,gjd->btgd", d_used, u)
    return base + scale[..., None] * resid


def _reads_above(src, layer):
    """A source above the reader (top/middle configuration, "A Systematic
    Study of Cross-Layer KV Sharing for Efficient LLM Inference", TL;DR:
    diagonal masking): its K/V for the current token does not exist yet."""
    return any(int(s) > layer for s in src[layer] if int(s) >= 0)


def layer_decode(src, w, layer, owner_k, owner_v, q, seq_len):
    """Decode output of ``layer`` under map (src, w): effective K/V, then
    attention; a layer reading a source above it skips the current position.
    Returns float64 [B, Hq, hd]."""
    k, v = effective_kv(src[layer], w[layer], owner_k, owner_v)
    return attend_decode(q, k, v, seq_len, exclude_current=_reads_above(src, layer))


def layer_prefill(src, w, layer, owner_k, owner_v, q, seq_len, causal=True):
    """Prefill-chunk output of ``layer`` under map (src, w)."""
    k, v = effective_kv(src[layer], w[layer], owner_k, owner_v)
    return attend_prefill(q, k, v, seq_len, causal=causal,
                          exclude_current=_reads_above(src, layer))
