"""Pins for the fp64 oracle of the factorized cache's write side (pair basis,
residual directions, encoder): a hand-derived token, closed forms of the
singular value decomposition, library rounding, and exact identities.  Each
would fail under a plausible mistake in the oracle (see
``test_planted_mistakes_are_caught_by_the_write_side_pins``)."""
import json
import os

import numpy as np
import torch

from oracle import attention as A
from oracle import factorize as Fz


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _orth_rows(k, n, seed):
    g = np.random.default_rng(seed)
    q, r = np.linalg.qr(g.standard_normal((n, k)))
    return (q * np.sign(np.diag(r))).T                  # [k, n], orthonormal rows


def _sign_norm(rows):
    rows = rows.copy()
    for i in range(rows.shape[0]):
        j = int(np.argmax(np.abs(rows[i])))
        if rows[i, j] < 0:
            rows[i] = -rows[i]
    return rows


# ----------------------------------------------------------------------------
# rounding helpers against torch's conversions
# ----------------------------------------------------------------------------

def test_rounding_matches_torch_conversions():
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 3))
    x32 = x.to(torch.float32)
    want_bf = x32.to(torch.bfloat16).double().numpy()
    want_h = x32.to(torch.float16).double().numpy()
    assert np.array_equal(Fz.round_bf16(x32.double().numpy()), want_bf)
    with np.errstate(over="ignore"):                 # beyond the half range: inf on both sides
        assert np.array_equal(Fz.round_fp16(x32.double().numpy()), want_h)
    # exact ties go to even
    assert Fz.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert Fz.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2 * 2.0 ** -7


# ----------------------------------------------------------------------------
# leading directions: closed forms
# ----------------------------------------------------------------------------

def check_svd_closed_form(leading=Fz.leading_directions):
    """rows = A diag(3, 2, 1) Q with orthonormal columns A and orthonormal rows
    Q: the leading directions are Q's rows in order (up to sign)."""
    n, hd = 50, 7
    a = _orth_rows(3, n, 1).T                          # [n, 3] orthonormal columns
    q = _orth_rows(3, hd, 2)
    rows = a @ np.diag([3.0, 2.0, 1.0]) @ q
    got = leading(rows, 3)
    return float(np.max(np.abs(got - _sign_norm(q))))


def test_leading_directions_closed_form():
    assert check_svd_closed_form() < 1e-12


def check_pair_basis_subspaces(pair_basis=Fz.pair_basis):
    """Layer a's rows span Q0, Q1 (singular values 4, 3), layer b's span Q2, Q3
    (2, 1), with junk rows past each sequence's count: rank 4 spans Q0..Q3,
    rank 2 spans Q0, Q1."""
    hd, n = 8, 40
    q = _orth_rows(4, hd, 5)
    a_cols = _orth_rows(4, n, 6).T
    xa = a_cols[:, :2] @ np.diag([4.0, 3.0]) @ q[:2]
    xb = a_cols[:, 2:] @ np.diag([2.0, 1.0]) @ q[2:]
    junk = np.full((1, 9, 1, hd), 1e3)
    xa = np.concatenate([xa[None, :, None, :], junk], axis=1)
    xb = np.concatenate([xb[None, :, None, :], junk], axis=1)
    err = 0.0
    for rank, want in ((4, q), (2, q[:2])):
        b = pair_basis(xa, xb, [n], rank)[0]
        err = max(err, float(np.max(np.abs(b.T @ b - want.T @ want))))
    return err


def test_pair_basis_spans_the_stacked_rows():
    assert check_pair_basis_subspaces() < 1e-10


def check_residual_basis_axes(residual_basis=Fz.residual_basis):
    """Owner rows bf16-exact in span(e0, e1); the layer adds energies 4, 3, 2, 1
    on e2..e5: the residual directions are e2..e5 in that order."""
    hd, n, R = 8, 60, 2
    g = np.random.default_rng(9)
    basis = np.eye(hd)[None, :R]
    owner = np.zeros((1, n, 1, hd))
    owner[0, :, 0, :R] = Fz.round_bf16(g.standard_normal((n, R)))
    cols = _orth_rows(4, n, 10).T
    extra = cols @ np.diag([4.0, 3.0, 2.0, 1.0])
    x = owner.copy()
    x[0, :, 0, R:R + 4] += extra
    u = residual_basis(x, owner, basis, [n], 4)[0]
    return float(np.max(np.abs(u - np.eye(hd)[R:R + 4])))


def test_residual_basis_of_axis_aligned_residual():
    assert check_residual_basis_axes() < 1e-10


# ----------------------------------------------------------------------------
# encoder: hand-derived token, exact identities
# ----------------------------------------------------------------------------

def check_quantize_token(golden, encode=Fz.encode):
    x = np.array(golden["x"])[None, None, None, :]
    basis = np.array(golden["basis"], dtype=np.float64)[None]
    ubasis = np.array(golden["ubasis"], dtype=np.float64)[None]
    err = 0.0
    for case in golden["cases"]:
        c, y, s, d = encode(x, x, basis, ubasis, np.array([[case["rank"]]]))
        err = max(err, float(np.max(np.abs(c[0, 0, 0] - golden["c"]))),
                  abs(float(s[0, 0, 0]) - case["s"]),
                  float(np.max(np.abs(d[0, 0, 0] - np.array(case["d"])))))
    return err


def test_golden_quantized_token(golden_dir):
    assert check_quantize_token(_load(golden_dir, "quantize_token.json")) == 0.0


def _random_layer(seed, B=2, T=40, Hkv=2, hd=16, R=4, Rm=6):
    g = np.random.default_rng(seed)
    basis = np.stack([Fz.leading_directions(g.standard_normal((50, hd)), R) for _ in range(Hkv)])
    ubasis = np.stack([Fz.leading_directions(g.standard_normal((50, hd)), Rm) for _ in range(Hkv)])
    x = g.standard_normal((B, T, Hkv, hd))
    owner = x + 0.3 * g.standard_normal((B, T, Hkv, hd))
    rank = g.integers(0, Rm + 1, size=(B, T))
    return x, owner, basis, ubasis, rank


def check_quantizer_properties(encode=Fz.encode):
    """Per token: |y_j - s d_j| <= s/2 for j < r (round to nearest), the
    largest |y_j| maps to +-127, codes past the rank are zero, and negating
    the rows negates coefficients and codes."""
    x, owner, basis, ubasis, rank = _random_layer(11)
    c, y, s, d = encode(x, owner, basis, ubasis, rank)
    bad = 0
    rmax = y.shape[-1]
    for b in range(x.shape[0]):
        for t in range(x.shape[1]):
            r = int(rank[b, t])
            for g in range(x.shape[2]):
                if r == 0:
                    bad += int(s[b, t, g] != 0 or np.any(d[b, t, g] != 0))
                    continue
                yy, dd, ss = y[b, t, g, :r], d[b, t, g, :r], s[b, t, g]
                bad += int(np.any(np.abs(yy - ss * dd) > ss / 2 * (1 + 1e-12)))
                bad += int(np.max(np.abs(dd)) != 127)
                bad += int(np.any(d[b, t, g, r:rmax] != 0))
    c2, _, s2, d2 = encode(-x, -owner, basis, ubasis, rank)
    bad += int(not np.array_equal(c2, -c)) + int(not np.array_equal(d2, -d))
    bad += int(not np.array_equal(s2, s))
    return bad


def test_quantizer_properties():
    assert check_quantizer_properties() == 0


def check_reconstruction_identity(encode=Fz.encode):
    """With orthonormal residual directions, the rebuilt row misses the
    original by the quantization error inside the kept directions and the
    residual outside them, orthogonally:
    ||x^ - x||^2 = ||s d - y_{<r}||^2 + ||e - U_{<r}^T y_{<r}||^2."""
    x, owner, basis, ubasis, rank = _random_layer(12)
    c, y, s, d = encode(x, owner, basis, ubasis, rank)
    xh = A.factorized_kv(c, basis, s, d, ubasis, rank)
    e = Fz.residual_rows(x, owner, basis)
    worst = 0.0
    for b in range(x.shape[0]):
        for t in range(x.shape[1]):
            r = int(rank[b, t])
            for g in range(x.shape[2]):
                u = ubasis[g, :r]
                yy = y[b, t, g, :r]
                lhs = np.sum((xh[b, t, g] - x[b, t, g]) ** 2)
                rhs = (np.sum((s[b, t, g] * d[b, t, g, :r] - yy) ** 2)
                       + np.sum((e[b, t, g] - u.T @ yy) ** 2))
                worst = max(worst, abs(lhs - rhs))
    return worst


def test_reconstruction_error_identity():
    assert check_reconstruction_identity() < 1e-9


# ----------------------------------------------------------------------------
# the pins catch planted mistakes
# ----------------------------------------------------------------------------

def test_planted_mistakes_are_caught_by_the_write_side_pins(golden_dir):
    tok = _load(golden_dir, "quantize_token.json")

    def floor_codes(x, xo, b, u, r):
        c, y, s, d = Fz.encode(x, xo, b, u, r)
        safe = np.where(s > 0, s, 1.0)[..., None]
        d = np.where(d != 0, np.clip(np.floor(y / safe), -127, 127), 0).astype(np.int64)
        return c, y, s, d

    assert check_quantize_token(tok, floor_codes) >= 1
    assert check_quantizer_properties(floor_codes) > 0

    def scale_128(x, xo, b, u, r):
        c, y, s, d = Fz.encode(x, xo, b, u, r)
        s2 = Fz.round_fp16(np.where(s > 0, np.max(np.abs(np.where(d != 0, y, 0)), axis=-1), 0) / 128)
        safe = np.where(s2 > 0, s2, 1.0)[..., None]
        d2 = np.where(d != 0, np.clip(np.rint(y / safe), -127, 127), 0).astype(np.int64)
        return c, y, s2, d2

    assert check_quantize_token(tok, scale_128) > 0

    def rank_off_by_one(x, xo, b, u, r):
        return Fz.encode(x, xo, b, u, np.asarray(r) + 1)

    assert check_quantize_token(tok, rank_off_by_one) > 0

    def residual_plus(x, xo, b, u, r):          # x + cB instead of x - cB
        c = Fz.coefficients(xo, b)
        x2 = A.f64(x) + 2 * np.einsum("btgi,gid->btgd", c, A.f64(b))
        return Fz.encode(x2, xo, b, u, r)

    assert check_reconstruction_identity(residual_plus) > 1e-3

    def smallest_first(rows, k):                # eigh order: ascending
        _, vecs = np.linalg.eigh(A.f64(rows).T @ A.f64(rows))
        return _sign_norm(vecs[:, :k].T)

    assert check_svd_closed_form(smallest_first) > 0.1

    def largest_unordered(rows, k):             # right subspace, wrong order
        return Fz.leading_directions(rows, k)[::-1]

    assert check_svd_closed_form(largest_unordered) > 0.1

    def one_layer_only(xa, xb, lens, rank):
        return Fz.pair_basis(xa, xa, lens, rank)

    assert check_pair_basis_subspaces(one_layer_only) > 0.1

    def lens_ignored(xa, xb, lens, rank):
        return Fz.pair_basis(xa, xb, [A.f64(xa).shape[1]], rank)

    assert check_pair_basis_subspaces(lens_ignored) > 0.1

    def no_owner_projection(x, xo, b, lens, rmax):
        return Fz.residual_basis(x, np.zeros_like(A.f64(xo)), b, lens, rmax)

    assert check_residual_basis_axes(no_owner_projection) > 0.1
