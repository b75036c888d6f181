"""Pins for the Layer Absorb / layer-selection oracle (CPU only).

The ISPA page (section 2, stage 2 "Layer Absorb") fixes the ridge objective and its closed form;
"Dynamic Layer Selection" ranks layers by reconstruction error. These tests pin `oracle.absorb` to a
hand-worked example, the normal equations evaluated on the raw rows, ridge regression as augmented
least squares (a QR route that never forms a Gram matrix), exact rationals, limits, linearity,
chunking invariance, optimality and exhaustive search for the ranking.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import ispa_inputs as inputs
from oracle import absorb as oab
from oracle import attention as oatt
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(seed, n=60, d=12, scale=1.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, d)) * np.exp(-np.linspace(0, 2, d)) * scale
    b = 0.7 * a + 0.3 * a[:, rng.permutation(d)] + 0.2 * rng.standard_normal((n, d)) * scale
    w = rng.standard_normal((d, d)) / np.sqrt(d)
    return a, b, w


def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "ridge_hand_2x2.json")))
    a, b, w = (np.array(g[k], dtype=np.float64) for k in ("a_loc", "a_full", "w"))
    st = oab.grams(a, b)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, g["lam"])
    np.testing.assert_allclose(dw, np.array([[float(Fraction(x)) for x in r] for r in g["dw"]]), atol=1e-15)
    assert abs(oab.layer_error_rows(a, b, w, dw) - float(Fraction(g["eps"]))) < 1e-14
    assert abs(oab.layer_error_stats(st["G"], st["C"], st["H"], w, dw) - float(Fraction(g["eps"]))) < 1e-14
    assert abs(oab.reference_energy(st["F"], w) - float(Fraction(g["ref"]))) < 1e-14
    assert abs(oab.objective(a, b, w, dw, g["lam"]) - float(Fraction(g["objective"]))) < 1e-14


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("lam", [1e-2, 1.0])
def test_normal_equations_from_rows(seed, lam):
    """P-5: (A_loc^T A_loc + lam I) dW = A_loc^T (A_full - A_loc) W, evaluated from the rows."""
    a, b, w = _rows(seed)
    st = oab.grams(a, b)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, lam)
    lhs = a.T @ (a @ dw) + lam * dw
    rhs = a.T @ ((b - a) @ w)
    assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-10


def test_stat_definitions_from_rows():
    a, b, w = _rows(4, n=30, d=5)
    st = oab.grams(a, b)
    n, d = a.shape
    G = np.zeros((d, d)); X = np.zeros((d, d)); F = np.zeros((d, d)); C = np.zeros((d, d)); H = np.zeros((d, d))
    for r in range(n):
        G += np.outer(a[r], a[r]); X += np.outer(a[r], b[r]); F += np.outer(b[r], b[r])
        C += np.outer(a[r], b[r] - a[r]); H += np.outer(b[r] - a[r], b[r] - a[r])
    for k, ref in (("G", G), ("X", X), ("F", F), ("C", C), ("H", H)):
        np.testing.assert_allclose(st[k], ref, atol=1e-12)
    np.testing.assert_allclose(st["C"], st["X"] - st["G"], atol=1e-12)
    np.testing.assert_allclose(st["H"], st["F"] - st["X"] - st["X"].T + st["G"], atol=1e-12)


def test_zero_when_full_equals_local():
    """P-6: A_full = A_loc gives C = 0 and dW = 0."""
    a, _, w = _rows(5)
    st = oab.grams(a, a)
    assert np.all(st["C"] == 0.0)
    assert np.all(oab.ridge_delta_w(st["G"], st["C"], w, 1e-2) == 0.0)


def test_large_lambda_limit():
    """P-7: dW -> 0 as lam -> inf, and lam dW -> C W."""
    a, b, w = _rows(6)
    st = oab.grams(a, b)
    cw = st["C"] @ w
    prev = None
    for lam in (1e2, 1e4, 1e6, 1e8):
        dw = oab.ridge_delta_w(st["G"], st["C"], w, lam)
        rel = np.linalg.norm(lam * dw - cw) / np.linalg.norm(cw)
        if prev is not None:
            assert rel < prev
        prev = rel
    assert prev < 1e-5
    assert np.linalg.norm(oab.ridge_delta_w(st["G"], st["C"], w, 1e8)) < 1e-6 * np.linalg.norm(w)


@pytest.mark.parametrize("seed,n,d", [(7, 60, 12), (8, 10, 12), (9, 128, 128)])
def test_augmented_least_squares(seed, n, d):
    """P-8: ridge = least squares on [A_loc; sqrt(lam) I] against [D W; 0] (QR, no Gram matrix)."""
    a, b, w = _rows(seed, n=n, d=d)
    lam = 1e-2
    st = oab.grams(a, b)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, lam)
    aug = np.vstack([a, np.sqrt(lam) * np.eye(d)])
    rhs = np.vstack([(b - a) @ w, np.zeros((d, d))])
    ref, *_ = np.linalg.lstsq(aug, rhs, rcond=None)
    tol = 1e-8 if n > d else 1e-6
    assert np.linalg.norm(dw - ref) / np.linalg.norm(ref) < tol


def test_linearity_in_w():
    """P-9: dW is linear in W, and dW(I) = (G + lam I)^-1 C."""
    a, b, w1 = _rows(10)
    _, _, w2 = _rows(11)
    st = oab.grams(a, b)
    f = lambda w: oab.ridge_delta_w(st["G"], st["C"], w, 0.1)
    np.testing.assert_allclose(f(2.0 * w1 - 3.0 * w2), 2.0 * f(w1) - 3.0 * f(w2), atol=1e-10)
    d = w1.shape[0]
    dwi = f(np.eye(d))
    np.testing.assert_allclose((st["G"] + 0.1 * np.eye(d)) @ dwi, st["C"], atol=1e-10)


def test_chunking_and_row_order():
    """P-10: statistics summed over chunks equal those of the stacked rows, in any row order,
    and a save/restore between chunks changes nothing."""
    a, b, _ = _rows(12, n=90)
    whole = oab.grams(a, b)
    chunks = [(a[i:i + 30], b[i:i + 30]) for i in (0, 30, 60)]
    acc = oab.accumulate(chunks)
    perm = np.random.default_rng(0).permutation(90)
    shuf = oab.grams(a[perm], b[perm])
    first = oab.accumulate(chunks[:2])
    saved = {k: v.copy() for k, v in first.items()}
    resumed = {k: saved[k] + oab.grams(*chunks[2])[k] for k in saved}
    for k in whole:
        np.testing.assert_allclose(acc[k], whole[k], atol=1e-12)
        np.testing.assert_allclose(shuf[k], whole[k], atol=1e-12)
        np.testing.assert_allclose(resumed[k], whole[k], atol=1e-12)


def test_optimality_and_error_bounds():
    """P-11: J(dW*) <= J(dW* + delta), and 0 <= eps(dW*) <= ||D W||^2 = eps(0)."""
    a, b, w = _rows(13)
    lam = 1e-2
    st = oab.grams(a, b)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, lam)
    j0 = oab.objective(a, b, w, dw, lam)
    rng = np.random.default_rng(1)
    for s in (1e-1, 1e-3, 1e-5):
        delta = rng.standard_normal(dw.shape) * s
        assert oab.objective(a, b, w, dw + delta, lam) >= j0
    eps = oab.layer_error_rows(a, b, w, dw)
    eps0 = oab.layer_error_rows(a, b, w, np.zeros_like(dw))
    np.testing.assert_allclose(eps0, np.sum(((b - a) @ w) ** 2), rtol=1e-13)
    assert 0.0 <= eps <= eps0


@pytest.mark.parametrize("seed", [14, 15])
def test_error_identity(seed):
    """P-12: eps from the summed statistics equals eps on the rows, for the optimum and any dW."""
    a, b, w = _rows(seed)
    st = oab.grams(a, b)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, 1e-2)
    for cand in (dw, np.zeros_like(dw), np.random.default_rng(seed).standard_normal(dw.shape) * 0.1):
        e_rows = oab.layer_error_rows(a, b, w, cand)
        e_stats = oab.layer_error_stats(st["G"], st["C"], st["H"], w, cand)
        assert abs(e_rows - e_stats) <= 1e-11 * max(1.0, e_rows)


@pytest.mark.parametrize("seed", [16, 17])
@pytest.mark.parametrize("lam", [1e-2, 3.0])
def test_error_at_the_optimum(seed, lam):
    """At the closed-form optimum (G + lam I) dW = C W =: B, so <dW, G dW> = <dW, B> - lam ||dW||^2 and
    eps = <W, H W> - <dW, B> - lam ||dW||^2; with L L^T = G + lam I and Y = L^-1 B, <dW, B> = ||Y||_F^2
    (B^T (L L^T)^-1 B = (L^-1 B)^T (L^-1 B)), and <W, H W> = <(F + G) - (X + X^T), W W^T>. The error on
    the rows must come out of these three terms; a wrong sign or a missing lam term fails."""
    a, b, w = _rows(seed)
    st = oab.grams(a, b)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, lam)
    B = st["C"] @ w
    L = np.linalg.cholesky(st["G"] + lam * np.eye(st["G"].shape[0]))
    Y = np.linalg.solve(L, B)
    H = (st["F"] + st["G"]) - (st["X"] + st["X"].T)
    np.testing.assert_allclose(H, st["H"], rtol=0, atol=1e-12 * np.abs(st["F"]).max())
    wh = np.sum(H * (w @ w.T))
    e_rows = oab.layer_error_rows(a, b, w, dw)
    assert abs(np.sum(Y * Y) - np.sum(dw * B)) <= 1e-11 * np.sum(dw * B)
    assert abs((wh - np.sum(Y * Y) - lam * np.sum(dw * dw)) - e_rows) <= 1e-10 * max(1.0, e_rows)
    # away from the optimum the shortcut does not hold
    off = dw * 1.1
    assert abs(oab.layer_error_rows(a, b, w, off) - (wh - np.sum(off * B) - lam * np.sum(off * off))) > 1e-6


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_brute_force(seed):
    """P-13: d <= 4 with small-integer A_loc, D, W and lam = 1, solved in exact rationals."""
    rng = np.random.default_rng(seed)
    n, d = 6, 3 + seed % 2
    a = rng.integers(-3, 4, size=(n, d))
    dm = rng.integers(-2, 3, size=(n, d))
    w = rng.integers(-2, 3, size=(d, d))
    exact = brute.ridge_exact(a.tolist(), dm.tolist(), w.tolist(), Fraction(1))
    st = oab.grams(a, a + dm)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, 1.0)
    np.testing.assert_allclose(dw, np.array([[float(x) for x in r] for r in exact]), atol=1e-14)


def test_ranking_brute_force():
    """P-14: the selected layers are the K smallest errors (exhaustive search), ties to lower index."""
    rng = np.random.default_rng(2)
    for trial in range(20):
        n = int(rng.integers(3, 9))
        k = int(rng.integers(1, n))
        eps = rng.integers(0, 5, size=n).astype(float)   # many ties
        sel, mask = oab.rank_layers(eps, k)
        best = brute.select_k_smallest(list(eps), k)
        assert tuple(sorted(sel.tolist())) == best
        assert mask.sum() == k and all(mask[i] for i in sel)
        assert list(eps[sel]) == sorted(eps[sel])


def test_ranking_nan_goes_last():
    sel, _ = oab.rank_layers(np.array([np.nan, 1.0, 0.5]), 2)
    assert sel.tolist() == [2, 1]


def test_chain_on_attention_outputs_tiny():
    """End-to-end on workload 1 (fp64 throughout): attention -> statistics -> dW -> eps.
    Checks the normal equations and 0 <= eps <= eps(0) on real attention outputs."""
    inp = inputs.attention_inputs(1)
    out = oatt.dual_stream(inp)
    w = inputs.weight(1, 0).astype(np.float64)
    st = oab.grams(out["A_loc"], out["A_full"])
    dw = oab.ridge_delta_w(st["G"], st["C"], w, 1e-2)
    a, b = out["A_loc"], out["A_full"]
    res = a.T @ (a @ dw) + 1e-2 * dw - a.T @ ((b - a) @ w)
    assert np.linalg.norm(res) / np.linalg.norm(a.T @ ((b - a) @ w)) < 1e-9
    eps = oab.layer_error_rows(a, b, w, dw)
    assert 0 <= eps <= oab.layer_error_rows(a, b, w, 0 * dw)
    assert abs(eps - oab.layer_error_stats(st["G"], st["C"], st["H"], w, dw)) < 1e-10 * eps
