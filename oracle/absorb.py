"""Oracle for Layer Absorb and layer selection (fp64, plain definitions).

TEST INFRASTRUCTURE (see `oracle/__init__.py`): importable only by tests, the smoke check and the
benchmark's CPU baseline.

Source: ISPA summary page, section 2 "Framework Core", stage 2 "Layer Absorb":
  objective      min_dW || A_loc (W + dW) - A_full W ||^2 + lam || dW ||^2     (first display eq.)
  closed form    dW = (A_loc^T A_loc + lam I)^-1 A_loc^T (A_full - A_loc) W     (second display eq.)
and "Dynamic Layer Selection": after the warmup every layer is ranked by its reconstruction error
eps and the lowest-error layers become local-attention layers (L-Layers).

Readings of points the page leaves open:
  * the norm on the matrices is the squared Frobenius norm (the closed form is exactly the Frobenius
    ridge solution);
  * W is the attention output projection, y = A @ W, W in R^{d x d}, d = H * d_h;
  * the statistics are sums over all warmup rows (every chunk, no 1/N), so lam is absolute;
  * eps is the data term of the objective at the given dW, summed over the warmup rows:
    eps = || A_loc (W + dW) - A_full W ||_F^2, with ||A_full W||_F^2 as its natural reference;
  * exactly K layers convert, ascending eps, ties to the lower layer index.
"""
from __future__ import annotations

from typing import Dict, Iterable, Tuple

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def grams(a_loc: np.ndarray, a_full: np.ndarray) -> Dict[str, np.ndarray]:
    """Warmup statistics of one block of rows (sums over rows, float64).

    G = A_loc^T A_loc, X = A_loc^T A_full, F = A_full^T A_full, and, with D = A_full - A_loc,
    C = A_loc^T D (the right-hand-side factor of the closed form) and H = D^T D.
    """
    a = _f64(a_loc)
    b = _f64(a_full)
    dd = b - a
    return {"G": a.T @ a, "X": a.T @ b, "F": b.T @ b, "C": a.T @ dd, "H": dd.T @ dd}


def accumulate(chunks: Iterable[Tuple[np.ndarray, np.ndarray]]) -> Dict[str, np.ndarray]:
    """Statistics summed over the warmup chunks (each chunk a pair (A_loc, A_full))."""
    tot = None
    for a_loc, a_full in chunks:
        g = grams(a_loc, a_full)
        tot = g if tot is None else {k: tot[k] + g[k] for k in tot}
    return tot


def ridge_delta_w(G: np.ndarray, C: np.ndarray, W: np.ndarray, lam: float) -> np.ndarray:
    """Closed-form absorb update dW = (G + lam I)^-1 C W (LU solve, float64)."""
    G = _f64(G)
    d = G.shape[0]
    return np.linalg.solve(G + lam * np.eye(d), _f64(C) @ _f64(W))


def layer_error_rows(a_loc: np.ndarray, a_full: np.ndarray, W: np.ndarray, dW: np.ndarray) -> float:
    """eps = || A_loc (W + dW) - A_full W ||_F^2 evaluated on the rows themselves."""
    r = _f64(a_loc) @ (_f64(W) + _f64(dW)) - _f64(a_full) @ _f64(W)
    return float(np.sum(r * r))


def layer_error_stats(G: np.ndarray, C: np.ndarray, H: np.ndarray, W: np.ndarray,
                      dW: np.ndarray) -> float:
    """The same eps from the summed statistics.

    With R = A_loc dW - D W:  ||R||^2 = <dW, G dW> - 2 <dW, C W> + <W, H W>.
    """
    W = _f64(W)
    dW = _f64(dW)
    return float(np.sum(dW * (_f64(G) @ dW)) - 2.0 * np.sum(dW * (_f64(C) @ W))
                 + np.sum(W * (_f64(H) @ W)))


def reference_energy(F: np.ndarray, W: np.ndarray) -> float:
    """|| A_full W ||_F^2 = <W, F W> (the scale eps is naturally compared against)."""
    W = _f64(W)
    return float(np.sum(W * (_f64(F) @ W)))


def objective(a_loc, a_full, W, dW, lam) -> float:
    """The absorb objective of the page at a given dW (data term + lam ||dW||_F^2)."""
    return layer_error_rows(a_loc, a_full, W, dW) + lam * float(np.sum(_f64(dW) ** 2))


def rank_layers(eps: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Select the k layers with the lowest eps (stable: ties go to the lower index).

    Returns (selected indices in ascending-eps order, boolean L-Layer mask).
    """
    eps = np.asarray(eps, dtype=np.float64)
    key = np.where(np.isnan(eps), np.inf, eps)
    order = np.argsort(key, kind="stable")
    sel = order[:k]
    mask = np.zeros(eps.shape[0], dtype=bool)
    mask[sel] = True
    return sel, mask
