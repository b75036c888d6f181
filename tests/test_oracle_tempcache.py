"""Pins for the TempCache exact-merge oracle (CPU only).

FAST-AR summary page, section 2 part A "TempCache", Lemma 5.1: merging identical keys loses nothing
when the group's values are averaged and the merged key's logit is shifted by the log of the group
size. The biased attention oracle is pinned to the plain attention oracle (itself pinned against
loops and hand cases) through that identity, through two more identities of the softmax (a bias
that is constant over the keys shifts the LSE and leaves the output; a bias of -1e300 removes a key)
and through per-head masks; the merge is pinned against exact rational means and identities.
"""
from fractions import Fraction

import numpy as np
import pytest

import ispa_inputs as inputs
from oracle import attention as oatt
from oracle import tempcache as otc


def _dup_keys(rng, n_groups, H, dh, max_size):
    sizes = rng.integers(1, max_size + 1, size=n_groups)
    base = rng.standard_normal((n_groups, H, dh))
    labels = rng.permutation(np.repeat(np.arange(n_groups), sizes))   # members scattered in the cache
    k = base[labels]
    v = rng.standard_normal((labels.size, H, dh))
    return k, v, labels


@pytest.mark.parametrize("seed,H,dh,max_size", [(0, 2, 8, 4), (1, 3, 16, 7), (2, 1, 4, 1)])
def test_lemma_merged_equals_duplicated(seed, H, dh, max_size):
    rng = np.random.default_rng(seed)
    k, v, labels = _dup_keys(rng, 23, H, dh, max_size)
    q = rng.standard_normal((9, H, dh))
    full = oatt.attention(q, k, v, 0.7)
    off, mem = inputs.csr_from_labels(labels)
    m = otc.merge_groups(k, v, off, mem)
    got = otc.attention_biased(q, m["k"], m["v"], 0.7, m["bias"])
    np.testing.assert_allclose(got["A"], full["A"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse"], full["lse"], rtol=0, atol=1e-12)
    # without the shift the merged cache under-weights the groups: the identity needs the ln m term
    if max_size > 1:
        plain = otc.attention_biased(q, m["k"], m["v"], 0.7, None)
        assert np.max(np.abs(plain["lse"] - full["lse"])) > 1e-3


def test_constant_bias_shifts_lse_only():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal(s) for s in ((5, 3, 8), (11, 3, 8), (11, 3, 8)))
    base = oatt.attention(q, k, v, 0.5)
    c = np.array([0.3, -2.0, 7.5])
    got = otc.attention_biased(q, k, v, 0.5, np.repeat(c[:, None], 11, axis=1))   # [H, n]
    np.testing.assert_allclose(got["A"], base["A"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse"], base["lse"] + c[:, None], rtol=0, atol=1e-12)
    shared = otc.attention_biased(q, k, v, 0.5, np.full(11, 1.25))                   # [n]
    np.testing.assert_allclose(shared["lse"], base["lse"] + 1.25, rtol=0, atol=1e-12)


def test_per_head_mask_removes_keys():
    # a very negative bias on key j of head h drops that key from head h only
    rng = np.random.default_rng(6)
    H, n = 3, 13
    q, k, v = (rng.standard_normal(s) for s in ((4, H, 8), (n, H, 8), (n, H, 8)))
    keep = rng.random((H, n)) < 0.6
    keep[:, 0] = True
    bias = np.where(keep, 0.0, -1e300)
    got = otc.attention_biased(q, k, v, 0.9, bias)
    for h in range(H):
        idx = np.nonzero(keep[h])[0]
        ref = oatt.attention(q[:, h:h + 1], k[idx][:, h:h + 1], v[idx][:, h:h + 1], 0.9)
        np.testing.assert_allclose(got["A"][:, h * 8:(h + 1) * 8], ref["A"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(got["lse"][h], ref["lse"][0], rtol=0, atol=1e-12)


def test_merge_exact_rational_means():
    rng = np.random.default_rng(8)
    k = rng.integers(-20, 21, size=(10, 2, 3)).astype(np.float64)
    v = rng.integers(-20, 21, size=(10, 2, 3)).astype(np.float64)
    labels = np.array([2, 0, 1, 2, 0, 2, 3, 1, 2, 4])
    off, mem = inputs.csr_from_labels(labels)
    m = otc.merge_groups(k, v, off, mem)
    for g in range(5):
        rows = [t for t in range(10) if labels[t] == g]
        assert m["count"][g] == len(rows)
        assert m["bias"][g] == pytest.approx(float(np.log(len(rows))), abs=0)
        for h in range(2):
            for c in range(3):
                want_k = sum(Fraction(int(k[t, h, c])) for t in rows) / len(rows)
                want_v = sum(Fraction(int(v[t, h, c])) for t in rows) / len(rows)
                assert abs(Fraction(m["k"][g, h, c]) - want_k) <= Fraction(1, 2 ** 48)
                assert abs(Fraction(m["v"][g, h, c]) - want_v) <= Fraction(1, 2 ** 48)


def test_merge_identities():
    rng = np.random.default_rng(9)
    k, v = rng.standard_normal((7, 2, 4)), rng.standard_normal((7, 2, 4))
    off, mem = inputs.csr_from_labels(np.arange(7))       # singletons: nothing changes
    m = otc.merge_groups(k, v, off, mem)
    np.testing.assert_array_equal(m["k"], k)
    np.testing.assert_array_equal(m["v"], v)
    np.testing.assert_array_equal(m["bias"], np.zeros(7))
    # identical keys with an 8-bit significand (bf16 values: sums of five are exact) merge to
    # themselves exactly
    kk = np.repeat(inputs.round_bf16(k[:1].astype(np.float32)).astype(np.float64), 5, axis=0)
    off, mem = inputs.csr_from_labels(np.zeros(5, dtype=np.int64))
    m = otc.merge_groups(kk, v[:5], off, mem)
    np.testing.assert_array_equal(m["k"][0], kk[0])
    with pytest.raises(ValueError):
        otc.merge_groups(k, v, np.array([0, 0, 7]), np.arange(7))


def test_dual_stream_zero_bias_is_plain_and_merged_history_is_exact():
    inp = inputs.static_history_case(3, n_heads=2, head_dim=16, n_q=20, n_sink=8, n_cur=24,
                                     n_frames=5, frame_tokens=12, static_frac=0.5)
    plain = oatt.dual_stream(inp)
    zero = otc.dual_stream_biased(inp, {})
    for name in ("A_loc", "A_full", "lse_loc", "lse_hist", "lse_full"):
        np.testing.assert_array_equal(zero[name], plain[name])
    off, mem = inp["hist_groups"]
    assert off[-1] == 60 and off.size - 1 == 6 + 5 * 6     # 6 static groups of 5, 30 singletons
    m = otc.merge_groups(inp["hist_k"], inp["hist_v"], off, mem)
    merged = dict(inp, hist_k=m["k"], hist_v=m["v"])
    got = otc.dual_stream_biased(merged, {"hist": m["bias"]})
    for name in ("A_loc", "A_full", "lse_loc", "lse_hist", "lse_full"):
        np.testing.assert_allclose(got[name], plain[name], rtol=0, atol=1e-12)


def test_csr_from_labels():
    off, mem = inputs.csr_from_labels(np.array([1, 0, 1, 2, 0]))
    assert off.tolist() == [0, 2, 4, 5]
    assert mem.tolist() == [1, 4, 0, 2, 3]
