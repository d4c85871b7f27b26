"""fp64 reference for the token router's statistics and rank choice.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "DepthWeave-KV: Smarter KV Cache Compression by Sharing Across Layers
and Adapting Per Token", Core Mechanism (a router reads attention statistics
-- entropy and peak scores -- to give instruction-carrying and
retrieval-critical tokens higher-rank residuals and compress generic ones,
online at every generation step) and Key Concepts (the more peaked a token's
attention, i.e. the lower its entropy, the more important the token and the
higher its reconstruction rank).  The page gives neither formulas nor
thresholds.  Readings (also listed with the design notes):

* Statistics of one decode query (a sequence's current token, one query
  head): the entropy H = -sum_t p_t ln p_t of its attention distribution over
  the keys it sees, and its peak probability max_t p_t.
* The router, per sequence, over one or more sets of statistics (layers):
  h = the mean over sets and heads of H / ln(n), n the keys the query saw
  (h = 0 when n <= 1), and p = the largest peak.  The token gets
  rank_focused when h < entropy_focused or p >= peak_focused, rank_mid when
  h < entropy_diffuse, else rank_diffuse (clamped to [0, Rmax]).
"""
from __future__ import annotations

import numpy as np

from .attention import f64


def attention_stats(q, k, seq_len, scale=None, exclude_current=False):
    """Entropy (nats) and peak probability of each decode query's attention:
    q [B, Hq, hd], k [B, T, Hkv, hd] -> [B, Hq, 2] float64.  A query that sees
    no key gets (0, 0)."""
    q = f64(q)
    k = f64(k)
    B, Hq, hd = q.shape
    G = Hq // k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.zeros((B, Hq, 2))
    for b in range(B):
        n = int(seq_len[b]) - (1 if exclude_current else 0)
        if n <= 0:
            continue
        for h in range(Hq):
            z = scale * (k[b, :n, h // G, :] @ q[b, h])
            p = np.exp(z - z.max())
            p /= p.sum()
            nz = p > 0
            out[b, h, 0] = -np.sum(p[nz] * np.log(p[nz]))
            out[b, h, 1] = p.max()
    return out


def route_ranks(stats, n_keys, entropy_focused, entropy_diffuse, peak_focused,
                rank_focused, rank_mid, rank_diffuse, rmax=16):
    """Rank per sequence from statistics [S, B, Hq, 2] and the keys each query
    saw, n_keys [B].  Returns (ranks [B] int64, h [B] the mean normalized
    entropy, p [B] the largest peak)."""
    st = np.asarray(stats, dtype=np.float64)
    if st.ndim == 3:
        st = st[None]
    B = st.shape[1]
    ranks = np.zeros(B, dtype=np.int64)
    hs = np.zeros(B)
    ps = np.zeros(B)
    for b in range(B):
        n = int(n_keys[b])
        h = float(np.mean(st[:, b, :, 0])) / np.log(n) if n > 1 else 0.0
        p = float(np.max(st[:, b, :, 1]))
        if h < entropy_focused or p >= peak_focused:
            r = rank_focused
        elif h < entropy_diffuse:
            r = rank_mid
        else:
            r = rank_diffuse
        ranks[b] = min(max(int(r), 0), rmax)
        hs[b], ps[b] = h, p
    return ranks, hs, ps
