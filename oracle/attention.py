"""Oracle for the dual-stream attention outputs (fp64, plain definition).

TEST INFRASTRUCTURE (see `oracle/__init__.py`): importable only by tests, the smoke check and the
benchmark's CPU baseline.

Source: ISPA summary page, section 2 "Framework Core", stage 1 "Dual-Stream Warmup". During the
warmup the layer produces two attention outputs for the same queries:
  A_full  over all cached keys (sink, history and the current chunk),
  A_loc   over the local context only (the sink tokens and the current chunk).
The page's Decomposable Attention obtains both from one pass by tracking log-sum-exp (LSE) states
per branch and merging them afterwards; that is an exact rewriting, so the oracle computes each
output directly from its own key set and never merges.

Readings of points the page leaves open:
  * queries are the current-chunk tokens; no mask (full attention within the chunk, all cached keys
    visible);
  * softmax per head with scale tau (1/sqrt(d_h) in every workload); heads are concatenated into
    columns h*d_h + c of A;
  * the LSE of a key set X is the natural log of sum_{j in X} exp(tau q.k_j) (tau included);
  * an empty key set has LSE = -inf and output 0.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              block: int = 512) -> Dict[str, np.ndarray]:
    """Softmax attention of queries q over keys k / values v, per head, in float64.

    q: [n_q, H, d_h], k, v: [n_k, H, d_h]. Returns
      "A":   [n_q, H*d_h]  A[i, h*d_h + c] = sum_j softmax_j(tau q_ih.k_jh) v_jhc
      "lse": [H, n_q]      lse[h, i] = log sum_j exp(tau q_ih.k_jh)
    The score matrix is formed explicitly, `block` query rows at a time (memory only).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, H, dh = q.shape
    n_k = k.shape[0]
    A = np.zeros((n_q, H * dh), dtype=np.float64)
    lse = np.full((H, n_q), -np.inf, dtype=np.float64)
    if n_k == 0:
        return {"A": A, "lse": lse}
    for h in range(H):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for i0 in range(0, n_q, block):
            i1 = min(n_q, i0 + block)
            s = scale * (q[i0:i1, h, :] @ kh.T)            # scores [b, n_k]
            m = s.max(axis=1, keepdims=True)               # shift for a finite exp; cancels exactly
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            A[i0:i1, h * dh:(h + 1) * dh] = (e @ vh) / z
            lse[h, i0:i1] = (m + np.log(z))[:, 0]
    return {"A": A, "lse": lse}


def dual_stream(inp: Dict[str, np.ndarray], scale: float = None, rows=None) -> Dict[str, np.ndarray]:
    """Both warmup streams of one (layer, chunk), each from its own key set.

    `inp` holds "q", "sink_k/v", "cur_k/v", "hist_k/v" ([n, H, d_h]); `rows` optionally selects query
    rows (for sampled checks at full size). Returns A_loc, A_full [n_q, d], lse_loc, lse_hist,
    lse_full [H, n_q] and A_hist (attention over the history keys alone, 0 where empty).
    """
    if scale is None:
        scale = float(inp["scale"])
    q = inp["q"] if rows is None else inp["q"][rows]
    loc_k = np.concatenate([inp["sink_k"], inp["cur_k"]], axis=0)
    loc_v = np.concatenate([inp["sink_v"], inp["cur_v"]], axis=0)
    all_k = np.concatenate([loc_k, inp["hist_k"]], axis=0)
    all_v = np.concatenate([loc_v, inp["hist_v"]], axis=0)
    loc = attention(q, loc_k, loc_v, scale)
    hist = attention(q, inp["hist_k"], inp["hist_v"], scale)
    full = attention(q, all_k, all_v, scale)
    return {"A_loc": loc["A"], "A_full": full["A"], "A_hist": hist["A"],
            "lse_loc": loc["lse"], "lse_hist": hist["lse"], "lse_full": full["lse"]}
