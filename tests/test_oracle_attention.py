"""Pins for the attention oracle (CPU only).

Each test checks `oracle.attention` against something other than itself: hand-worked values, closed
forms, the log-sum-exp merge identity fixed by the ISPA page's Decomposable Attention (section 2,
stage 1), key-permutation invariance, and pure-Python brute force.
"""
import json
import math
import os

import numpy as np
import pytest

import ispa_inputs as inputs
from oracle import attention as oatt
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        return {"ln3": math.log(3.0), "ln4": math.log(4.0)}[x]
    return float(x)


def _arr(nested, shape_tail=None):
    def conv(o):
        if isinstance(o, list):
            return [conv(e) for e in o]
        return _num(o)
    a = np.array(conv(nested), dtype=np.float64)
    if a.size == 0 and shape_tail is not None:
        a = a.reshape((0,) + shape_tail)
    return a


def test_golden_two_key_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_hand_2key.json")))
    inp = {name: _arr(g[name], (1, 2)) for name in
           ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    out = oatt.dual_stream(inp, scale=g["scale"])
    np.testing.assert_allclose(out["A_loc"], _arr(g["a_loc"]), atol=1e-15)
    np.testing.assert_allclose(out["A_full"], _arr(g["a_full"]), atol=1e-14)
    np.testing.assert_allclose(out["lse_loc"], _arr(g["lse_loc"]), atol=1e-15)
    np.testing.assert_allclose(out["lse_hist"], _arr(g["lse_hist"]), atol=1e-15)
    np.testing.assert_allclose(out["lse_full"], _arr(g["lse_full"]), atol=1e-15)


def _small(seed, H=2, dh=8, n_q=7, ns=5, nc=6, nh=11, rho=None):
    return inputs.attention_case(seed, H, dh, n_q, ns, nc, nh, dtype="f32", rho=rho)


def _merge(A1, l1, A2, l2, dh):
    """LSE merge of two disjoint key sets (the Decomposable Attention identity)."""
    l = np.logaddexp(l1, l2)
    w1 = np.exp(l1 - l)
    w2 = np.exp(l2 - l)
    H = l.shape[0]
    rep = lambda w: np.repeat(w.T, dh, axis=1)   # [n_q, H*dh]
    A = rep(w1) * A1 + rep(w2) * A2
    return A, l


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_merge_identity_equals_single_pass(seed):
    """P-1: the local and history branches merged by LSE equal attention over all keys."""
    inp = _small(seed)
    out = oatt.dual_stream(inp)
    A, l = _merge(out["A_loc"], out["lse_loc"], out["A_hist"], out["lse_hist"], 8)
    np.testing.assert_allclose(l, out["lse_full"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(A, out["A_full"], rtol=0, atol=1e-12)


def test_local_branch_ignores_history():
    """P-2: A_loc and lse_loc depend only on the sink and current keys."""
    inp = _small(5)
    out1 = oatt.dual_stream(inp)
    inp2 = dict(inp)
    inp2["hist_k"] = inp["hist_k"] * 3.0 + 1.0
    inp2["hist_v"] = -inp["hist_v"]
    out2 = oatt.dual_stream(inp2)
    np.testing.assert_array_equal(out1["A_loc"], out2["A_loc"])
    np.testing.assert_array_equal(out1["lse_loc"], out2["lse_loc"])
    assert not np.allclose(out1["A_full"], out2["A_full"])


def test_empty_history():
    """Empty history: A_full = A_loc, lse_hist = -inf, lse_full = lse_loc."""
    inp = _small(6, nh=0)
    out = oatt.dual_stream(inp)
    np.testing.assert_array_equal(out["A_full"], out["A_loc"])
    np.testing.assert_array_equal(out["lse_full"], out["lse_loc"])
    assert np.all(np.isneginf(out["lse_hist"]))


def test_closed_form_equal_keys():
    """P-3: all keys equal k* -> A = mean of V and lse = tau <q, k*> + log n."""
    rng = np.random.default_rng(11)
    n, H, dh, tau = 37, 3, 16, 0.25
    q = rng.standard_normal((5, H, dh))
    kstar = rng.standard_normal((1, H, dh))
    k = np.repeat(kstar, n, axis=0)
    v = rng.standard_normal((n, H, dh))
    out = oatt.attention(q, k, v, tau)
    for h in range(H):
        np.testing.assert_allclose(out["A"][:, h * dh:(h + 1) * dh],
                                   np.broadcast_to(v[:, h].mean(axis=0), (5, dh)), atol=1e-13)
        np.testing.assert_allclose(out["lse"][h], tau * q[:, h] @ kstar[0, h] + math.log(n), atol=1e-12)


def test_closed_form_single_key_constant_v_zero_q():
    rng = np.random.default_rng(12)
    H, dh = 2, 4
    q = rng.standard_normal((3, H, dh))
    k1 = rng.standard_normal((1, H, dh))
    v1 = rng.standard_normal((1, H, dh))
    out = oatt.attention(q, k1, v1, 0.5)
    np.testing.assert_allclose(out["A"], np.broadcast_to(v1.reshape(1, -1), (3, H * dh)), atol=1e-15)
    np.testing.assert_allclose(out["lse"], 0.5 * np.einsum("ihc,hc->hi", q, k1[0]), atol=1e-14)
    # constant V -> A is that constant whatever the scores
    k = rng.standard_normal((19, H, dh))
    vc = np.full((19, H, dh), 2.5)
    np.testing.assert_allclose(oatt.attention(q, k, vc, 0.5)["A"], 2.5, atol=1e-14)
    # Q = 0 -> uniform weights: lse = log n exactly and A = mean of V
    v = rng.standard_normal((19, H, dh))
    o0 = oatt.attention(np.zeros((3, H, dh)), k, v, 0.5)
    np.testing.assert_allclose(o0["lse"], math.log(19), atol=1e-15)
    np.testing.assert_allclose(o0["A"][0], v.mean(axis=0).reshape(-1), atol=1e-14)


def test_split_invariance_and_key_permutation():
    """P-4: splitting the keys into sub-segments and merging in any order gives the same result."""
    rng = np.random.default_rng(13)
    H, dh, n = 2, 8, 41
    q = rng.standard_normal((6, H, dh))
    k = rng.standard_normal((n, H, dh)) * 2.0
    v = rng.standard_normal((n, H, dh))
    ref = oatt.attention(q, k, v, 0.3)
    cuts = [0, 7, 8, 25, n]
    parts = [oatt.attention(q, k[a:b], v[a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
    for order in ([0, 1, 2, 3], [3, 1, 0, 2]):
        A, l = parts[order[0]]["A"], parts[order[0]]["lse"]
        for i in order[1:]:
            A, l = _merge(A, l, parts[i]["A"], parts[i]["lse"], dh)
        np.testing.assert_allclose(A, ref["A"], atol=1e-12)
        np.testing.assert_allclose(l, ref["lse"], atol=1e-12)
    perm = rng.permutation(n)
    p = oatt.attention(q, k[perm], v[perm], 0.3)
    np.testing.assert_allclose(p["A"], ref["A"], atol=1e-13)
    np.testing.assert_allclose(p["lse"], ref["lse"], atol=1e-13)


def test_query_blocking_does_not_change_result():
    inp = _small(7, n_q=23)
    q, k, v = inp["q"], inp["cur_k"], inp["cur_v"]
    a = oatt.attention(q, k, v, 0.2, block=512)
    b = oatt.attention(q, k, v, 0.2, block=4)
    np.testing.assert_array_equal(a["lse"], b["lse"])
    np.testing.assert_allclose(a["A"], b["A"], atol=1e-15)


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_loops(seed):
    """P-13: 1-2 heads x 8 queries x 24 keys against pure-Python loops (math.exp, fsum)."""
    inp = inputs.attention_case(100 + seed, 2, 4, 8, 4, 8, 12, dtype="f32", scale=0.7)
    out = oatt.dual_stream(inp)
    loc_k = np.concatenate([inp["sink_k"], inp["cur_k"]])
    loc_v = np.concatenate([inp["sink_v"], inp["cur_v"]])
    all_k = np.concatenate([loc_k, inp["hist_k"]])
    all_v = np.concatenate([loc_v, inp["hist_v"]])
    tl = lambda a: a.astype(np.float64).tolist()
    for name, kk, vv, lname in (("A_loc", loc_k, loc_v, "lse_loc"), ("A_full", all_k, all_v, "lse_full"),
                                ("A_hist", inp["hist_k"], inp["hist_v"], "lse_hist")):
        A, lse = brute.attention_loops(tl(inp["q"]), tl(kk), tl(vv), 0.7)
        np.testing.assert_allclose(out[name], np.array(A).reshape(8, -1), atol=1e-14)
        np.testing.assert_allclose(out[lname], np.array(lse), atol=1e-14)


def test_ar1_generator_statistics():
    """The AR(1) key chain keeps N(0,1) marginals and lag-1 correlation rho (input recipe check)."""
    rng = np.random.default_rng(3)
    k = inputs.ar1_key_frames(rng, 12, 1, 32, frame_tokens=400).reshape(12, 400 * 32)
    assert abs(k.std() - 1.0) < 0.02
    c = np.mean(k[1:] * k[:-1]) / np.mean(k * k)
    assert abs(c - 0.95) < 0.01
