"""Oracle for the L-Layer steady state (plain definitions; exact or float64).

TEST INFRASTRUCTURE (see `oracle/__init__.py`): importable only by tests, the smoke check and the
benchmark's CPU baseline.

Source: ISPA summary page, section 2 "Framework Core", stage 3 "Memory-Efficient Inference": after
the warmup the K selected layers become L-Layers for every later frame. They evict their history
keys and values, attend to the local context only (sink tokens and the current chunk), and their
output projection uses the updated weights W_new = W + dW. The other N - K layers stay F-Layers:
full attention over the whole cache and the original W.

Readings of points the page leaves open:
  * the updated weights are stored at the model's precision, bf16: W_new = bf16(fp32(W + dW)), the
    sum taken in fp32 and rounded to nearest, ties to even; they are kept in the orientation of an
    nn.Linear weight, [d_out, d_in], so that y = A W_new^T;
  * the projection reads bf16 activations A [n, d_in] and writes bf16 outputs y [n, d_out]; the
    products are exact and the sum is the exact real sum (fp64 here), rounded once at the end;
  * eviction: an L-Layer keeps its sink and current-chunk keys and frees its whole history range;
    an F-Layer keeps everything.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np


def round_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values, round to nearest, ties to even.

    Written from the IEEE-754 rule: keep the upper 16 bits of the binary32 pattern and add one unit
    of the kept part when the dropped 16 bits exceed half a unit, or equal half a unit and the kept
    part is odd. NaN stays NaN (quiet, sign kept); overflow rounds to infinity by the same rule.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    r = (hi + up.astype(np.uint64)).astype(np.uint64)
    nan = np.isnan(f)
    r = np.where(nan, (hi | 0x0040), r)     # quiet NaN with the same sign and payload top bits
    return r.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def apply_delta(w, dw, w_is_linear_weight: bool = False) -> np.ndarray:
    """Updated weights of an L-Layer as bf16 bits in nn.Linear orientation [d_out, d_in].

    w, dw: float32 arrays of the same orientation: [d_in, d_out] with y = A W, or, with
    w_is_linear_weight, [d_out, d_in] with y = A W^T. The sum is one fp32 addition per element.
    """
    w32 = np.asarray(w, dtype=np.float32)
    d32 = np.asarray(dw, dtype=np.float32)
    s = (w32 + d32).astype(np.float32)
    if not w_is_linear_weight:
        s = s.T
    return round_to_bf16_bits(np.ascontiguousarray(s))


def project(a, w_linear) -> np.ndarray:
    """y = A W^T in float64 from exact inputs: a [n, d_in], w_linear [d_out, d_in] (float values)."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w_linear, dtype=np.float64).T


def layer_plan(is_l_layer: Sequence[bool], n_sink: int, n_hist: int, n_cur: int) -> Dict[str, object]:
    """Per-layer key ranges after the warmup, in cache order [sink | history | current].

    Returns for every layer the kept history length (0 for an L-Layer, n_hist for an F-Layer), the
    keys its attention reads, and the total number of evicted key/value tokens.
    """
    keep: List[int] = []
    keys: List[int] = []
    for flag in is_l_layer:
        kh = 0 if flag else int(n_hist)
        keep.append(kh)
        keys.append(int(n_sink) + kh + int(n_cur))
    evicted = sum(int(n_hist) for flag in is_l_layer if flag)
    return {"hist_kept": keep, "keys": keys, "evicted_tokens": evicted}
