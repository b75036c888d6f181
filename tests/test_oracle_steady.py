"""Pins for the L-Layer steady-state oracle (CPU only).

The ISPA page (section 2, stage 3 "Memory-Efficient Inference") fixes what an L-Layer does after
the warmup: it drops its history keys, attends to sink + current chunk only, and projects with
W + dW. These tests pin `oracle.steady` to the IEEE round-to-nearest-even rule (hand cases and a
brute-force nearest-value search), to projections whose result is known in closed form (identity,
permutation, exact integer brute force), to the eviction bookkeeping worked by hand, and to the
absorb oracle: on the warmup rows the L-Layer's output misses A_full W by exactly the layer error.
"""
import numpy as np
import pytest

from oracle import absorb as oab
from oracle import steady as ost


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


# (binary32 pattern, bf16 pattern) fixed by round-to-nearest-ties-to-even on a 16-bit cut
ROUND_CASES = [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # tie, kept part even: down
    (0x3F818000, 0x3F82),   # tie, kept part odd: up
    (0x3F808001, 0x3F81),   # above half: up
    (0x3F807FFF, 0x3F80),   # below half: down
    (0xBFC00000, 0xBFC0),   # -1.5 exact
    (0xBF818000, 0xBF82),   # negative tie, odd: away from zero in magnitude
    (0x7F7FFFFF, 0x7F80),   # largest finite rounds up to +inf
    (0x7F7F8000, 0x7F80),   # tie at the top, odd: +inf
    (0x7F7F7FFF, 0x7F7F),   # just below the tie: stays finite
    (0x7F800000, 0x7F80),   # +inf
    (0xFF800000, 0xFF80),   # -inf
    (0x80000000, 0x8000),   # -0
    (0x00000001, 0x0000),   # smallest subnormal: down to +0
    (0x00008000, 0x0000),   # subnormal tie, even: down
    (0x00018000, 0x0002),   # subnormal tie, odd: up
]


@pytest.mark.parametrize("src,want", ROUND_CASES)
def test_round_cases(src, want):
    assert int(ost.round_to_bf16_bits(_f32(src))[0]) == want


def test_round_nan_stays_nan():
    b = ost.round_to_bf16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(np.isnan(ost.bf16_bits_to_f64(b)))


def test_round_is_nearest_bf16_by_search():
    # brute force over the two neighbouring bf16 values, compared as exact float64 numbers
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    x = np.concatenate([x, (np.arange(1, 4000, dtype=np.uint32) << 15 | 0x3F800000).view(np.float32)])
    got = ost.bf16_bits_to_f64(ost.round_to_bf16_bits(x))
    u = x.view(np.uint32)
    lo_bits = (u >> 16).astype(np.uint16)
    hi_bits = (lo_bits.astype(np.uint32) + 1).astype(np.uint16)
    lo = ost.bf16_bits_to_f64(lo_bits)
    hi = ost.bf16_bits_to_f64(hi_bits)
    xv = x.astype(np.float64)
    dlo, dhi = np.abs(xv - lo), np.abs(hi - xv)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo_bits & 1) == 1))
    want = np.where(pick_hi, hi, lo)
    assert np.array_equal(got, want)


def test_apply_delta_orientation_and_exact_cases():
    rng = np.random.default_rng(3)
    d_in, d_out = 6, 4
    w = ost.bf16_bits_to_f64(ost.round_to_bf16_bits(rng.standard_normal((d_in, d_out)).astype(np.float32)))
    w = w.astype(np.float32)                      # bf16-representable
    zero = np.zeros_like(w)
    out = ost.apply_delta(w, zero)                # [d_out, d_in]
    assert out.shape == (d_out, d_in)
    assert np.array_equal(ost.bf16_bits_to_f64(out), w.T.astype(np.float64))
    # the linear-weight orientation is the transpose of the other
    out_lin = ost.apply_delta(w.T.copy(), zero.T.copy(), w_is_linear_weight=True)
    assert np.array_equal(out_lin, out)
    # dW = W doubles every weight: exact in both formats (an exponent step)
    got = ost.bf16_bits_to_f64(ost.apply_delta(w, w.copy()))
    np.testing.assert_array_equal(got, (2.0 * w.astype(np.float64)).T)
    # dW = -W gives exact zeros
    assert not np.any(ost.bf16_bits_to_f64(ost.apply_delta(w, -w)))


def test_apply_delta_within_half_ulp_of_exact_sum():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((32, 24)).astype(np.float32)
    dw = (1e-3 * rng.standard_normal((32, 24))).astype(np.float32)
    got = ost.bf16_bits_to_f64(ost.apply_delta(w, dw)).T
    exact = w.astype(np.float64) + dw.astype(np.float64)
    # fp32 sum (half an fp32 ulp) then bf16 rounding (half a bf16 ulp = 2^-8 relative at most)
    assert np.all(np.abs(got - exact) <= np.abs(exact) * (2.0 ** -8 + 2.0 ** -23) + 1e-38)


def test_project_closed_forms():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((7, 5))
    np.testing.assert_array_equal(ost.project(a, np.eye(5)), a)
    perm = rng.permutation(5)
    p = np.eye(5)[perm]                           # row r of W^T selects column perm[r] of A
    np.testing.assert_array_equal(ost.project(a, p), a[:, perm])
    np.testing.assert_array_equal(ost.project(a, 2.0 * np.eye(5)), 2.0 * a)


def test_project_integer_brute_force():
    rng = np.random.default_rng(9)
    a = rng.integers(-9, 10, size=(4, 6))
    wl = rng.integers(-9, 10, size=(3, 6))
    want = [[sum(int(a[i, k]) * int(wl[j, k]) for k in range(6)) for j in range(3)] for i in range(4)]
    np.testing.assert_array_equal(ost.project(a, wl), np.array(want, dtype=np.float64))


def test_layer_plan_by_hand():
    plan = ost.layer_plan([True, False, True, False], n_sink=10, n_hist=100, n_cur=30)
    assert plan["hist_kept"] == [0, 100, 0, 100]
    assert plan["keys"] == [40, 140, 40, 140]
    assert plan["evicted_tokens"] == 200
    empty = ost.layer_plan([], 1, 2, 3)
    assert empty == {"hist_kept": [], "keys": [], "evicted_tokens": 0}


def test_l_layer_output_misses_full_output_by_the_layer_error():
    # on the warmup rows, || A_loc (W + dW) - A_full W ||_F^2 is the layer error eps of the absorb
    rng = np.random.default_rng(21)
    n, d = 80, 10
    a_loc = rng.standard_normal((n, d))
    a_full = 0.8 * a_loc + 0.3 * rng.standard_normal((n, d))
    w = rng.standard_normal((d, d)) / np.sqrt(d)
    st = oab.grams(a_loc, a_full)
    dw = oab.ridge_delta_w(st["G"], st["C"], w, 0.05)
    y_l = ost.project(a_loc, (w + dw).T)          # L-Layer: local attention output, updated weights
    y_f = ost.project(a_full, w.T)                # F-Layer target on the same rows
    eps = oab.layer_error_rows(a_loc, a_full, w, dw)
    assert abs(float(np.sum((y_l - y_f) ** 2)) - eps) <= 1e-10 * max(1.0, eps)
    # and the update never makes it worse than keeping W (dW = 0 is feasible)
    assert eps <= float(np.sum((ost.project(a_loc, w.T) - y_f) ** 2)) + 1e-12
