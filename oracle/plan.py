"""Reference semantics of a layer -> source sharing map.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
* CLA page ("Reducing Transformer Key-Value Cache Size with Cross-Layer
  Attention"), Methodology: some layers compute new K/V, the others reuse it.
  A reusing layer computes no K/V of its own, so it can never be a source:
  every source named in the map must be a layer that owns its K/V.
* Same page, Key Results / Abstract: sharing between adjacent layers (CLA2)
  halves the cache.
* DepthGraft page, Abstract: deep-layer K/V is rebuilt from stride-aligned
  shallow/middle source pairs and the cache shrinks by roughly one third.
* "A Systematic Study of Cross-Layer KV Sharing for Efficient LLM
  Inference", TL;DR and Abstract: the bottom configurations take K/V from
  lower layers; the top/middle ones pair queries with K/V of upper layers,
  and inference with them relies on diagonal masking.  Reading: when a
  layer runs, a source above it has not yet produced the current token's
  K/V, so such a layer's query sees only earlier positions (the diagonal of
  its causal mask is removed); see ``excludes_current``.

Map encoding: ``src`` [L, 2] ints (-1 = unused second entry), ``w`` [L, 2]
float weights.  A layer owns its K/V iff its row is ((l, 1.0), (-1, *)).
"""
from __future__ import annotations

import math

OK = "ok"
ERR_MAP = "map"                 # malformed row: bad index, weight, or self-row shape
ERR_NOT_SOURCE = "not_source"   # a source that does not own K/V (a chain)
ERR_UNSUPPORTED = "unsupported"  # more sources than a factorized plan takes


def owns(src, w, l) -> bool:
    return int(src[l][0]) == l and int(src[l][1]) < 0 and float(w[l][0]) == 1.0


def check(src, w, max_sources_factorized=None) -> str:
    """Classify a map: OK or the first violated rule, scanning layers in order
    and, within a layer, the rules in the order: index range and weight
    finiteness (ERR_MAP), more than one source in a factorized plan
    (ERR_UNSUPPORTED), a self-reference that is not the plain owner row
    (ERR_MAP), a source that does not own K/V (ERR_NOT_SOURCE).  Sources above
    their reader (top/middle configurations) are allowed."""
    L = len(src)
    if L == 0:
        return ERR_MAP
    for l in range(L):
        row = [int(s) for s in src[l]]
        if not (0 <= row[0] < L):
            return ERR_MAP
        if not (row[1] == -1 or 0 <= row[1] < L):
            return ERR_MAP
        n = 1 if row[1] < 0 else 2
        for j in range(n):
            if not math.isfinite(float(w[l][j])):
                return ERR_MAP
        if max_sources_factorized is not None and n > max_sources_factorized:
            return ERR_UNSUPPORTED
        if l in row[:n] and not owns(src, w, l):
            return ERR_MAP
        for j in range(n):
            if not owns(src, w, row[j]):
                return ERR_NOT_SOURCE
    return OK


def owner_layers(src, w):
    return [l for l in range(len(src)) if owns(src, w, l)]


def slots(src, w):
    """Owner slot of every owner layer: its rank among owners, ascending."""
    return {l: i for i, l in enumerate(owner_layers(src, w))}


def layer_sources(src, w, l):
    """[(source layer, slot, weight)] for layer l, in row order."""
    sl = slots(src, w)
    out = []
    for j in range(2):
        s = int(src[l][j])
        if s >= 0:
            out.append((s, sl[s], float(w[l][j])))
    return out


def excludes_current(src, w, l) -> bool:
    """Whether layer l reads a source above it (a top/middle configuration):
    that source writes the current token's K/V only after layer l has run,
    so layer l's query attends to earlier positions only."""
    return any(int(s) > l for s in src[l] if int(s) >= 0)


def last_owner_layer(src, w) -> int:
    """The deepest layer that writes cache entries.  Layers above it own no
    K/V, so a prompt's non-final tokens need not run them (DepthGraft
    abstract: prefill can complete early)."""
    own = owner_layers(src, w)
    return own[-1] if own else -1


def cache_fraction(src, w) -> float:
    """Cached layers / all layers: the cache size relative to no sharing."""
    return len(owner_layers(src, w)) / len(src)
