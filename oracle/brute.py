"""Brute-force evaluations for tiny inputs: pure-Python loops and exact rationals.

TEST INFRASTRUCTURE (see `oracle/__init__.py`). These routines re-derive the ISPA quantities with
no NumPy linear algebra at all, so that the fp64 oracle can be pinned against them:
  * `attention_loops`  softmax attention by explicit loops over heads, queries and keys (ISPA page,
    section 2 stage 1: A_loc over sink+current keys, A_full over all keys);
  * `ridge_exact`      the closed-form Layer Absorb update (section 2 stage 2) in exact rational
    arithmetic, by Gauss-Jordan elimination on (A_loc^T A_loc + lam I) X = A_loc^T D W;
  * `select_k_smallest` layer selection by exhaustive search over all K-subsets.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction
from typing import List, Sequence, Tuple


def attention_loops(q, k, v, scale) -> Tuple[List[List[List[float]]], List[List[float]]]:
    """q: [n_q][H][d_h], k, v: [n_k][H][d_h] nested sequences. Returns (A[n_q][H][d_h], lse[H][n_q])."""
    n_q, H, dh = len(q), len(q[0]), len(q[0][0])
    n_k = len(k)
    A = [[[0.0] * dh for _ in range(H)] for _ in range(n_q)]
    lse = [[-math.inf] * n_q for _ in range(H)]
    for h in range(H):
        for i in range(n_q):
            if n_k == 0:
                continue
            s = [scale * math.fsum(q[i][h][c] * k[j][h][c] for c in range(dh)) for j in range(n_k)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            lse[h][i] = m + math.log(z)
            for c in range(dh):
                A[i][h][c] = math.fsum(w[j] * v[j][h][c] for j in range(n_k)) / z
    return A, lse


def _matmul(a, b):
    n, m, p = len(a), len(b), len(b[0])
    return [[sum((a[i][t] * b[t][j] for t in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def _transpose(a):
    return [list(r) for r in zip(*a)]


def ridge_exact(a_loc: Sequence[Sequence[int]], d_mat: Sequence[Sequence[int]],
                w: Sequence[Sequence[int]], lam: Fraction) -> List[List[Fraction]]:
    """Exact dW = (A^T A + lam I)^-1 A^T D W for small integer/rational A, D = A_full - A_loc, W."""
    A = [[Fraction(x) for x in r] for r in a_loc]
    D = [[Fraction(x) for x in r] for r in d_mat]
    Wm = [[Fraction(x) for x in r] for r in w]
    At = _transpose(A)
    M = _matmul(At, A)
    n = len(M)
    for i in range(n):
        M[i][i] += Fraction(lam)
    R = _matmul(_matmul(At, D), Wm)
    p = len(R[0])
    aug = [M[i] + R[i] for i in range(n)]
    for col in range(n):
        piv = next(r for r in range(col, n) if aug[r][col] != 0)
        aug[col], aug[piv] = aug[piv], aug[col]
        pv = aug[col][col]
        aug[col] = [x / pv for x in aug[col]]
        for r in range(n):
            if r != col and aug[r][col] != 0:
                f = aug[r][col]
                aug[r] = [x - f * y for x, y in zip(aug[r], aug[col])]
    return [row[n:n + p] for row in aug]


def select_k_smallest(eps: Sequence[float], k: int) -> Tuple[int, ...]:
    """The K-subset with the smallest total eps; among equal totals the lexicographically first."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(eps)), k):
        s = math.fsum(eps[i] for i in comb)
        if best_sum is None or s < best_sum:
            best, best_sum = comb, s
    return best
