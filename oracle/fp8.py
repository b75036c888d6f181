"""Oracle for the FP8 (e4m3) form of the attention scores (plain definitions; exact or float64).

TEST INFRASTRUCTURE (see `oracle/__init__.py`): importable only by tests, the smoke check and the
benchmark's CPU baseline.

Source: ISPA summary page, section 4 "Experimental Results": ISPA is combined with W8A8
post-training quantisation (8-bit weights and activations) for its largest end-to-end speed-up. The
page gives no quantisation recipe, so everything below is a reading (parity unpinned as to the recipe;
the arithmetic of each step is pinned):
  * format: OCP FP8 E4M3 ("E4M3FN": sign, 4 exponent bits with bias 7, 3 mantissa bits, no
    infinities, the all-ones pattern S.1111.111 is NaN, largest finite 448);
  * encoding: round to nearest, ties to even; magnitudes beyond 448 saturate to +-448; NaN -> 0x7F;
  * scaling: one scale per head for queries and one per head for the keys of the whole cache,
    scale = absmax / 448 (1 where the head is all zero); codes = e4m3(fp32(x * fp32(1 / scale)));
  * attention: the scores use the dequantised values q = e4m3_value * scale_q, k = e4m3_value *
    scale_k with exact products; values and probabilities stay at bf16 (only the score product is in
    FP8), so the FP8 attention oracle is the plain attention oracle on dequantised Q and K;
  * attention with an FP8 value product as well: the values are quantised per head over the whole cache
    like the keys, and the oracle is the plain attention oracle on dequantised Q, K and V. The device also
    rounds each probability to e4m3 before the value product; that rounding depends on the running
    maximum of an online softmax, which a plain definition does not have, so it is not part of the oracle
    (parity unpinned as to the probability rounding; `p_rounding_sigma` gives the spread it causes under a
    rounding model, for tolerances);
  * statistics: the attention outputs A_loc and A_full (rows [n, d], d = H * d_h) are quantised per
    head like the keys; G, X, F are the Gram sums of the dequantised rows (exact products), so the
    FP8 statistics oracle is the plain one on dequantised rows.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 values of e4m3 codes (uint8); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def _positive_table():
    codes = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: all finite non-negative codes
    return codes, e4m3_decode(codes)


def e4m3_encode(x) -> np.ndarray:
    """e4m3 codes of float values: nearest representable value, ties to the even mantissa; saturate
    at +-448; NaN -> 0x7F; the sign of zero is kept."""
    v = np.asarray(x, dtype=np.float64)
    codes, vals = _positive_table()
    a = np.abs(v)
    a_sat = np.minimum(np.nan_to_num(a, nan=0.0), E4M3_MAX)
    # index of the largest table value <= a, and the next one above
    lo = np.clip(np.searchsorted(vals, a_sat, side="right") - 1, 0, len(vals) - 1)
    hi = np.minimum(lo + 1, len(vals) - 1)
    d_lo = a_sat - vals[lo]
    d_hi = vals[hi] - a_sat
    lo_even = (codes[lo] & 1) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even & (hi != lo))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    out = np.where(np.signbit(v), mag | 0x80, mag).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), out).astype(np.uint8)


def head_scales(x) -> np.ndarray:
    """Per-head scale absmax / 448 of x [n, H, d] (float32; 1 for an all-zero head)."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float64)), axis=(0, 2)) if np.size(x) else np.zeros(np.shape(x)[1])
    s = (a / E4M3_MAX).astype(np.float32)
    return np.where(s > 0, s, np.float32(1.0)).astype(np.float32)


def quantize(x, scale) -> np.ndarray:
    """e4m3 codes of x [n, H, d] with per-head scales: e4m3(fp32(x * fp32(1 / scale)))."""
    x32 = np.asarray(x, dtype=np.float32)
    inv = (np.float32(1.0) / np.asarray(scale, dtype=np.float32)).astype(np.float32)
    y = (x32 * inv[None, :, None]).astype(np.float32)
    return e4m3_encode(y)


def dequantize(codes, scale) -> np.ndarray:
    """float64 values e4m3_value * scale of codes [n, H, d]."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[None, :, None]


def dual_stream_fp8(inp: Dict[str, np.ndarray], q_codes, q_scale, k_codes: Dict[str, np.ndarray], k_scale,
                    scale: float = None, rows=None, v_codes: Dict[str, np.ndarray] = None,
                    v_scale=None) -> Dict[str, np.ndarray]:
    """The dual-stream outputs with the scores taken from dequantised e4m3 queries and keys, and the
    values as given or, with `v_codes` / `v_scale`, dequantised e4m3 values. `k_codes` and `v_codes` map
    "sink", "cur", "hist" to codes; one key scale and one value scale per head for the whole cache."""
    from . import attention as oatt
    deq = dict(inp)
    deq["q"] = dequantize(q_codes, q_scale)
    for name in ("sink", "cur", "hist"):
        deq[name + "_k"] = dequantize(k_codes[name], k_scale)
        if v_codes is not None:
            deq[name + "_v"] = dequantize(v_codes[name], v_scale)
    return oatt.dual_stream(deq, scale=scale if scale is not None else float(inp["scale"]), rows=rows)


def p_rounding_sigma(q, keys, values, scale: float, rows=None) -> np.ndarray:
    """Standard deviation of each output element [n_q, H*d_h] that rounding every probability to e4m3
    causes, under the model of independent rounding errors uniform over half a spacing: a probability
    p = exp(s - max) >= 2^-6 (normal) is off by p * u with u uniform in +-2^-4 (std 2^-4 / sqrt(3)); a
    subnormal one by an absolute error uniform in +-2^-10. Exact float64 probabilities relative to the
    true maximum are used (the device's running maximum is never above it, so its probabilities are never
    smaller and this overstates the subnormal part). keys / values [n_k, H, d_h]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    if rows is not None:
        q = q[rows]
    n_q, H, dh = q.shape
    out = np.zeros((n_q, H * dh))
    for h in range(H):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        err = np.where(p >= 2.0 ** -6, p * 2.0 ** -4, 2.0 ** -10) / np.sqrt(3.0)
        L = p.sum(axis=1, keepdims=True)
        out[:, h * dh:(h + 1) * dh] = np.sqrt((err / L) ** 2 @ (v[:, h, :] ** 2))
    return out


def grams_fp8(loc_codes, loc_scale, full_codes, full_scale, head_dim: int) -> Dict[str, np.ndarray]:
    """G, X, F of dequantised e4m3 rows [n, d] with per-head scales ([d / head_dim] each)."""
    from . import absorb as oab
    n, d = np.shape(loc_codes)
    H = d // head_dim
    a = dequantize(np.reshape(loc_codes, (n, H, head_dim)), loc_scale).reshape(n, d)
    b = dequantize(np.reshape(full_codes, (n, H, head_dim)), full_scale).reshape(n, d)
    return oab.grams(a, b)
