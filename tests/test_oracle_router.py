"""Pins for the fp64 router oracle (oracle.router): a hand-derived two-key
entropy, closed forms (uniform attention, one key, a dominant key), a library
entropy routine, bounds, and hand-made router cases; each fails under the
planted mistakes at the end."""
import json
import math
import os

import numpy as np
from scipy.stats import entropy as scipy_entropy

from oracle import router as R


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def check_two_key_stats(golden, stats=R.attention_stats):
    two = _load(os.path.dirname(golden["_path"]), "two_key_softmax.json")
    q = np.array(two["q"])[None, None, :]
    k = np.array(two["k"])[None, :, None, :]
    st = stats(q, k, [2])
    return max(abs(st[0, 0, 0] - golden["two_key"]["entropy"]),
               abs(st[0, 0, 1] - golden["two_key"]["peak"]))


def _golden(golden_dir):
    g = _load(golden_dir, "router_token.json")
    g["_path"] = os.path.join(golden_dir, "router_token.json")
    return g


def test_two_key_entropy_and_peak(golden_dir):
    assert check_two_key_stats(_golden(golden_dir)) < 1e-12


def check_closed_forms(stats=R.attention_stats):
    """Equal keys: H = ln n, peak 1/n.  One key: (0, 1).  A dominant key
    (score gap 60 nats): H ~ 0, peak ~ 1.  The current position excluded:
    n - 1 keys."""
    g = np.random.default_rng(1)
    err = 0.0
    for n in (2, 5, 64):
        q = g.standard_normal((1, 2, 8))
        k = np.repeat(g.standard_normal((1, 1, 1, 8)), n, axis=1)
        st = stats(q, k, [n])
        err = max(err, float(np.max(np.abs(st[0, :, 0] - math.log(n)))),
                  float(np.max(np.abs(st[0, :, 1] - 1.0 / n))))
        st = stats(q, k, [n], exclude_current=True)
        want = math.log(n - 1) if n > 1 else 0.0
        err = max(err, float(np.max(np.abs(st[0, :, 0] - want))))
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = 1.0
    k = np.zeros((1, 3, 1, 4)); k[0, 1, 0, 0] = 120.0        # z = 60 for key 1
    st = stats(q, k, [3])
    err = max(err, abs(st[0, 0, 1] - 1.0), abs(st[0, 0, 0]))
    st = stats(q, k[:, :1], [1])
    err = max(err, abs(st[0, 0, 0]), abs(st[0, 0, 1] - 1.0))
    return err


def test_closed_forms():
    assert check_closed_forms() < 1e-9


def check_against_scipy(stats=R.attention_stats):
    """Random queries and keys (GQA, ragged lengths): entropy equals
    scipy.stats.entropy of the softmax probabilities, built here with
    scipy.special.softmax; peak equals their maximum; 0 <= H <= ln n."""
    from scipy.special import softmax
    g = np.random.default_rng(2)
    B, T, Hq, Hkv, hd = 2, 30, 4, 2, 8
    q = g.standard_normal((B, Hq, hd)) * 2
    k = g.standard_normal((B, T, Hkv, hd))
    lens = [30, 7]
    st = stats(q, k, lens)
    err = 0.0
    for b in range(B):
        for h in range(Hq):
            p = softmax(k[b, :lens[b], h // 2] @ q[b, h] / math.sqrt(hd))
            err = max(err, abs(st[b, h, 0] - scipy_entropy(p)), abs(st[b, h, 1] - p.max()))
            assert -1e-12 <= st[b, h, 0] <= math.log(lens[b]) + 1e-12
    return err


def test_stats_match_scipy_entropy():
    assert check_against_scipy() < 1e-12


def check_router_cases(golden, route=R.route_ranks):
    th = golden["thresholds"]
    bad = 0
    for c in golden["router_cases"]:
        n = c["n"]
        ln = math.log(n) if n > 1 else 1.0
        st = np.zeros((1, 1, 2, 2))
        st[0, 0, :, 0] = np.array(c["h_norm"]) * ln
        st[0, 0, :, 1] = c["peak"]
        r, _, _ = route(st, [n], th["entropy_focused"], th["entropy_diffuse"], c["peak_focused"],
                        th["rank_focused"], th["rank_mid"], th["rank_diffuse"])
        bad += int(r[0] != c["rank"])
    return bad


def test_router_cases(golden_dir):
    assert check_router_cases(_golden(golden_dir)) == 0


def test_router_averages_sets_and_clamps():
    """Two sets average like one set holding both; ranks clamp to [0, Rmax]."""
    st = np.zeros((2, 1, 1, 2))
    st[0, 0, 0] = (0.1 * math.log(8), 0.2)
    st[1, 0, 0] = (0.5 * math.log(8), 0.2)
    r, h, _ = R.route_ranks(st, [8], 0.31, 0.7, 0.9, 40, 8, -3)
    assert abs(h[0] - 0.3) < 1e-12 and r[0] == 16
    r, _, _ = R.route_ranks(st, [8], 0.29, 0.3, 0.9, 40, 8, -3)
    assert r[0] == 0


def test_planted_mistakes_are_caught_by_the_router_pins(golden_dir):
    g = _golden(golden_dir)

    def log2_entropy(q, k, seq_len, scale=None, exclude_current=False):
        st = R.attention_stats(q, k, seq_len, scale, exclude_current)
        st[..., 0] /= math.log(2)
        return st

    assert check_two_key_stats(g, log2_entropy) > 1e-3
    assert check_closed_forms(log2_entropy) > 1e-3

    def unscaled(q, k, seq_len, scale=None, exclude_current=False):
        return R.attention_stats(q, k, seq_len, 1.0, exclude_current)

    assert check_two_key_stats(g, unscaled) > 1e-3
    assert check_against_scipy(unscaled) > 1e-3

    def inverted(st, n, ef, ed, pf, rf, rm, rd, rmax=16):     # high entropy -> high rank
        return R.route_ranks(st, n, ef, ed, pf, rd, rm, rf, rmax)

    assert check_router_cases(g, inverted) > 0

    def unnormalized(st, n, ef, ed, pf, rf, rm, rd, rmax=16):  # H not divided by ln n
        return R.route_ranks(st, [math.e] * len(n), ef, ed, pf, rf, rm, rd, rmax)

    assert check_router_cases(g, unnormalized) > 0

    def peak_ignored(st, n, ef, ed, pf, rf, rm, rd, rmax=16):
        return R.route_ranks(st, n, ef, ed, 2.0, rf, rm, rd, rmax)

    assert check_router_cases(g, peak_ignored) > 0
