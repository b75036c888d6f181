"""Oracle for the TempCache exact merge of duplicate keys (fp64, plain definitions).

TEST INFRASTRUCTURE (see `oracle/__init__.py`): importable only by tests, the smoke check and the
benchmark's CPU baseline.

Source: FAST-AR summary page ("Sintesi Tecnica: FAST-AR", gist.science), section 2 "Componenti
Core", part A "TempCache", the bullet on its theoretical basis (Lemma 5.1): a group of identical
keys can be replaced by one key without any error when the group's values are averaged and the
logit of the merged key is shifted by the group size. Written out for one query q and a group of m
keys equal to k with values v_1 .. v_m:

    sum_{r<=m} exp(tau q.k) v_r  =  exp(tau q.k + ln m) * mean_r(v_r),
    sum_{r<=m} exp(tau q.k)      =  exp(tau q.k + ln m),

so softmax attention over the original keys equals attention over the merged keys with an
additive logit bias ln m on the merged key, and the log-sum-exp is unchanged.

Readings of points the page leaves open:
  * groups are sets of token positions of one cache segment, the same for all heads (a token is
    merged as a whole row of keys and values); the merged key is the mean of the group's keys,
    which is the common key when the keys are identical (the exact case of the lemma; the page
    merges near-duplicates above a similarity threshold in practice, which is then approximate);
  * the shift is the natural log of the group size, added to tau q.k; a bias may also be given
    per head ([H, n]) so that callers can merge per head;
  * the similarity search that finds the groups (approximate nearest neighbours over hashes or
    quantised codes) is a separate method and not part of this oracle: groups are inputs.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def merge_groups(k, v, offsets, members) -> Dict[str, np.ndarray]:
    """Merge the token rows of each group: means of keys and values, count and ln(count).

    k, v: [n, H, d_h]; groups in compressed form: group g holds token indices
    members[offsets[g]:offsets[g+1]] (offsets non-decreasing, offsets[0] = 0; every group has at
    least one member). Returns "k", "v" [G, H, d_h] (float64 means), "count" [G] and "bias" [G]
    (natural log of the count).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    mem = np.asarray(members, dtype=np.int64)
    n_groups = off.shape[0] - 1
    H, dh = k.shape[1], k.shape[2]
    km = np.zeros((n_groups, H, dh), dtype=np.float64)
    vm = np.zeros((n_groups, H, dh), dtype=np.float64)
    count = np.zeros(n_groups, dtype=np.int64)
    for g in range(n_groups):
        rows = mem[off[g]:off[g + 1]]
        if rows.size == 0:
            raise ValueError(f"group {g} is empty")
        km[g] = k[rows].mean(axis=0)
        vm[g] = v[rows].mean(axis=0)
        count[g] = rows.size
    return {"k": km, "v": vm, "count": count, "bias": np.log(count.astype(np.float64))}


def attention_biased(q, k, v, scale: float, bias=None, block: int = 512) -> Dict[str, np.ndarray]:
    """Softmax attention with an additive logit bias per key, per head, in float64.

    q: [n_q, H, d_h], k, v: [n_k, H, d_h]; bias: None (zero), [n_k] (all heads) or [H, n_k].
    Logit of key j for query i in head h: tau q_ih.k_jh + bias[h, j]. Returns "A" [n_q, H*d_h] and
    "lse" [H, n_q] (natural log of the sum of exp(logit); -inf and zero output for no keys).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, H, dh = q.shape
    n_k = k.shape[0]
    if bias is None:
        b = np.zeros((H, n_k), dtype=np.float64)
    else:
        b = np.asarray(bias, dtype=np.float64)
        b = np.broadcast_to(b, (H, n_k)) if b.ndim == 1 else b
    A = np.zeros((n_q, H * dh), dtype=np.float64)
    lse = np.full((H, n_q), -np.inf, dtype=np.float64)
    if n_k == 0:
        return {"A": A, "lse": lse}
    for h in range(H):
        for i0 in range(0, n_q, block):
            i1 = min(n_q, i0 + block)
            s = scale * (q[i0:i1, h, :] @ k[:, h, :].T) + b[h][None, :]
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            A[i0:i1, h * dh:(h + 1) * dh] = (e @ v[:, h, :]) / z
            lse[h, i0:i1] = (m + np.log(z))[:, 0]
    return {"A": A, "lse": lse}


def dual_stream_biased(inp: Dict[str, np.ndarray], bias: Optional[Dict[str, np.ndarray]] = None,
                       scale: float = None, rows=None) -> Dict[str, np.ndarray]:
    """Both warmup streams (local = sink + current, full = all three segments) with per-key biases.

    `inp` as for the plain dual stream ("q", "sink_k/v", "cur_k/v", "hist_k/v"); `bias` maps any of
    "sink", "cur", "hist" to a bias of that segment ([n] or [H, n]); a missing entry is zero.
    Returns A_loc, A_full [n_q, d] and lse_loc, lse_hist, lse_full [H, n_q].
    """
    if scale is None:
        scale = float(inp["scale"])
    bias = bias or {}
    q = inp["q"] if rows is None else inp["q"][rows]
    H = q.shape[1]

    def seg_bias(name):
        n = inp[name + "_k"].shape[0]
        b = bias.get(name)
        if b is None:
            return np.zeros((H, n), dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        return np.broadcast_to(b, (H, n)) if b.ndim == 1 else b

    loc_k = np.concatenate([inp["sink_k"], inp["cur_k"]], axis=0)
    loc_v = np.concatenate([inp["sink_v"], inp["cur_v"]], axis=0)
    loc_b = np.concatenate([seg_bias("sink"), seg_bias("cur")], axis=1)
    all_k = np.concatenate([loc_k, inp["hist_k"]], axis=0)
    all_v = np.concatenate([loc_v, inp["hist_v"]], axis=0)
    all_b = np.concatenate([loc_b, seg_bias("hist")], axis=1)
    loc = attention_biased(q, loc_k, loc_v, scale, loc_b)
    hist = attention_biased(q, inp["hist_k"], inp["hist_v"], scale, seg_bias("hist"))
    full = attention_biased(q, all_k, all_v, scale, all_b)
    return {"A_loc": loc["A"], "A_full": full["A"], "lse_loc": loc["lse"], "lse_hist": hist["lse"],
            "lse_full": full["lse"]}
