"""GPU parity of the TempCache exact merge (group merge kernel, biased dual-stream attention) against
the fp64 oracle (`oracle.tempcache`) on identical seeded inputs.

Gates: merged rows within one output rounding of the exact mean plus the fp32 summation error,
ln(count) within 2^-20; biased attention to the attention tolerances (bf16: A max-abs 1e-2 + 2^-7
|A|, rel-Frobenius 1e-2, LSE 1e-3; fp32: 1e-5); Lemma 5.1 on the GPU: attention over a merged
history with its log-count bias matches attention over the original history.
"""
import numpy as np
import pytest

import ispa_inputs as inputs
from oracle import attention as oatt
from oracle import tempcache as otc

from gpu_helpers import check_attention, empty_outputs, run_attn, to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _biases(rng, inp, layout, which, pad=0):
    H = inp["q"].shape[1]
    out = {}
    for name in which:
        n = inp[name + "_k"].shape[0]
        if layout == "shared":
            b = rng.uniform(-2.0, 2.0, n) + np.log(rng.integers(1, 9, n))
        else:
            b = rng.uniform(-2.0, 2.0, (H, n)) + np.log(rng.integers(1, 9, (H, n)))
        out[name] = b.astype(np.float32)
    return out


def _bias_dev(b, pad):
    torch = torch_mod()
    if b is None:
        return None
    if b.ndim == 1 or pad == 0:
        return torch.from_numpy(np.ascontiguousarray(b)).cuda()
    store = torch.full((b.shape[0], b.shape[1] + pad), float("nan"), dtype=torch.float32, device="cuda")
    store[:, :b.shape[1]] = torch.from_numpy(b).cuda()
    return store[:, :b.shape[1]]


def _run_biased(inp, bias, want_full=True, pad=0, dev=None):
    import kv_cache_attention_split_amd as ispa
    dt = inp["dtype"]
    if dev is None:
        dev = {k: to_dev(inp[k], dt) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    n_q, H, dh = inp["q"].shape
    out = empty_outputs(n_q, H, dh, dt, want_full)
    ispa.ispa_attn_dual_biased(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"],
                               dev["hist_k"], dev["hist_v"], float(inp["scale"]), out["a_loc"], out["a_full"],
                               out["lse_loc"], out["lse_hist"], out["lse_full"],
                               sink_bias=_bias_dev(bias.get("sink"), pad), cur_bias=_bias_dev(bias.get("cur"), pad),
                               hist_bias=_bias_dev(bias.get("hist"), pad))
    torch_mod().cuda.synchronize()
    return dev, out


# (dtype, H, d_h, n_q, sink, cur, hist, layout, biased segments, head-stride padding)
CASES = [
    ("bf16", 2, 128, 300, 40, 100, 333, "shared", ("sink", "cur", "hist"), 0),
    ("bf16", 2, 128, 257, 64, 64, 200, "per_head", ("hist",), 24),
    ("bf16", 3, 128, 130, 0, 75, 129, "per_head", ("cur", "hist"), 0),
    ("bf16", 3, 64, 200, 17, 70, 150, "per_head", ("sink", "cur", "hist"), 8),
    ("bf16", 2, 64, 100, 30, 30, 0, "shared", ("sink",), 0),
    ("f32", 2, 64, 150, 20, 45, 90, "shared", ("sink", "cur", "hist"), 0),
    ("f32", 2, 128, 129, 10, 33, 65, "per_head", ("hist",), 4),
]


@pytest.mark.parametrize("case", CASES)
def test_biased_attention_vs_oracle(case):
    dt, H, dh, n_q, ns, nc, nh, layout, which, pad = case
    _log(f"case: biased attention {case}")
    inp = inputs.attention_case(40 + n_q, n_heads=H, head_dim=dh, n_q=n_q, n_sink=ns, n_cur=nc, n_hist=nh,
                                dtype=dt)
    bias = _biases(np.random.default_rng(n_q + nh), inp, layout, which)
    _, out = _run_biased(inp, bias, pad=pad)
    ref = otc.dual_stream_biased(inp, bias)
    rep = check_attention(out, ref, dt)
    _log(f"   {rep}")


def test_biased_local_only_and_null_bias_is_plain():
    inp = inputs.attention_case(77, n_heads=2, head_dim=128, n_q=200, n_sink=32, n_cur=160, n_hist=96)
    bias = _biases(np.random.default_rng(3), inp, "shared", ("sink", "cur", "hist"))
    _, out = _run_biased(inp, bias, want_full=False)
    ref = otc.dual_stream_biased(inp, bias)
    check_attention(out, ref, "bf16")
    # no bias at all: bitwise the plain entry point
    dev, plain = run_attn(inp)
    _, none = _run_biased(inp, {}, dev=dev)
    torch = torch_mod()
    for k in ("a_loc", "a_full", "lse_loc", "lse_hist", "lse_full"):
        assert torch.equal(plain[k], none[k]), k


def test_biased_mask_drops_keys():
    # a bias of -1e30 removes a key: same result as attention over the kept keys only
    inp = inputs.attention_case(78, n_heads=2, head_dim=128, n_q=150, n_sink=0, n_cur=130, n_hist=140)
    rng = np.random.default_rng(5)
    keep = rng.random(140) < 0.5
    bias = {"hist": np.where(keep, 0.0, -1e30).astype(np.float32)}
    _, out = _run_biased(inp, bias)
    ref = oatt.dual_stream(dict(inp, hist_k=inp["hist_k"][keep], hist_v=inp["hist_v"][keep]))
    check_attention(out, ref, "bf16")


def _merge_gpu(k, v, off, mem, dt, pad=0):
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    G = off.size - 1
    H, dh = k.shape[1], k.shape[2]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    kd = to_dev(k.reshape(k.shape[0], H * dh), dt).reshape(k.shape[0], H, dh)
    vd = to_dev(v.reshape(v.shape[0], H * dh), dt).reshape(v.shape[0], H, dh)
    ko = torch.full((G, H * dh + pad), float("nan"), dtype=tdt, device="cuda")
    vo = torch.full((G + 2, H * dh + pad), float("nan"), dtype=tdt, device="cuda")
    bo = torch.full((G + 1,), float("nan"), dtype=torch.float32, device="cuda")
    kv = ko[:, :H * dh].reshape(G, H, dh) if pad == 0 else ko.as_strided((G, H, dh), (H * dh + pad, dh, 1))
    vv = vo[:G, :H * dh].reshape(G, H, dh) if pad == 0 else vo.as_strided((G, H, dh), (H * dh + pad, dh, 1))
    ispa.ispa_kv_merge(kd, vd, torch.from_numpy(off).cuda(), torch.from_numpy(mem).cuda(), kv, vv, bo[:G])
    torch.cuda.synchronize()
    assert torch.isnan(vo[G:]).all() and torch.isnan(bo[G:]).all(), "wrote past the last group"
    if pad:
        assert torch.isnan(ko[:, H * dh:]).all(), "wrote into the row padding"
    return to_host64(kv).reshape(G, H, dh), to_host64(vv).reshape(G, H, dh), to_host64(bo[:G])


def _check_merge(k, v, off, mem, got_k, got_v, got_b, dt):
    ref = otc.merge_groups(k, v, off, mem)
    cnt = ref["count"][:, None, None].astype(np.float64)
    for got, x, want in ((got_k, k, ref["k"]), (got_v, v, ref["v"])):
        absmean = otc.merge_groups(np.abs(x), np.abs(x), off, mem)["k"]
        if dt == "bf16":
            bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -22 * cnt * absmean + 1e-30
        else:
            bound = 2.0 ** -23 * np.abs(want) + 2.0 ** -22 * cnt * absmean + 1e-30
        assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) - bound))
    assert np.all(np.abs(got_b - ref["bias"]) <= 2.0 ** -20 * np.maximum(1.0, ref["bias"]))


@pytest.mark.parametrize("dt,H,dh,n,G,max_size,pad", [("bf16", 2, 128, 700, 300, 6, 0),
                                                     ("bf16", 12, 128, 2000, 1111, 3, 16),
                                                     ("bf16", 1, 8, 40, 40, 1, 0),
                                                     ("f32", 3, 64, 500, 123, 8, 8)])
def test_merge_vs_oracle(dt, H, dh, n, G, max_size, pad):
    _log(f"case: merge {dt} H={H} d_h={dh} rows={n} groups={G} pad={pad}")
    rng = np.random.default_rng(n + G)
    k = rng.standard_normal((n, H, dh)).astype(np.float32)
    v = rng.standard_normal((n, H, dh)).astype(np.float32)
    if dt == "bf16":
        k, v = inputs.round_bf16(k), inputs.round_bf16(v)
    sizes = rng.integers(1, max_size + 1, size=G)
    mem_all = rng.choice(n, size=int(sizes.sum()), replace=int(sizes.sum()) > n).astype(np.int32)
    off = np.zeros(G + 1, dtype=np.int32)
    off[1:] = np.cumsum(sizes)
    gk, gv, gb = _merge_gpu(k, v, off, mem_all, dt, pad)
    _check_merge(k, v, off, mem_all, gk, gv, gb, dt)


@pytest.mark.parametrize("dt,H,dh,n,G", [("bf16", 1, 128, 600, 12), ("f32", 1, 64, 400, 9),
                                         ("bf16", 2, 64, 700, 10), ("bf16", 1, 8, 300, 7)])
def test_merge_large_groups_narrow_rows(dt, H, dh, n, G):
    """Groups of 40 to 100 members on rows narrower than one pass of the wave (H * d_h < 512): the member
    indices of a group are read one per lane and broadcast, so every lane must take part in that read,
    also lanes whose columns lie past the row end; groups over 64 members cross a batch of indices."""
    _log(f"case: merge {dt} H={H} d_h={dh} rows={n} groups={G} of 40-100 members")
    rng = np.random.default_rng(7 * n + G)
    k = rng.standard_normal((n, H, dh)).astype(np.float32)
    v = rng.standard_normal((n, H, dh)).astype(np.float32)
    if dt == "bf16":
        k, v = inputs.round_bf16(k), inputs.round_bf16(v)
    sizes = rng.integers(40, 101, size=G)
    mem_all = rng.choice(n, size=int(sizes.sum()), replace=True).astype(np.int32)
    off = np.zeros(G + 1, dtype=np.int32)
    off[1:] = np.cumsum(sizes)
    gk, gv, gb = _merge_gpu(k, v, off, mem_all, dt)
    _check_merge(k, v, off, mem_all, gk, gv, gb, dt)


def test_merge_identical_keys_are_bitwise_and_bad_members_are_skipped():
    inp = inputs.static_history_case(5, n_heads=2, head_dim=64, n_q=8, n_sink=4, n_cur=8, n_frames=7,
                                     frame_tokens=40, static_frac=0.5)
    off, mem = inp["hist_groups"]
    gk, gv, gb = _merge_gpu(inp["hist_k"], inp["hist_v"], off, mem, "bf16")
    n_static = 20
    for g in range(n_static):
        first = mem[off[g]]
        np.testing.assert_array_equal(gk[g], inp["hist_k"][first].astype(np.float64))
    _check_merge(inp["hist_k"], inp["hist_v"], off, mem, gk, gv, gb, "bf16")
    # a member outside [0, n) contributes zero and is never read; an empty group gets zero rows and
    # bias -inf
    n = inp["hist_k"].shape[0]
    bad_off = np.array([0, 3, 3, 4, 7], dtype=np.int32)
    bad_mem = np.array([5, -1, n, 9, 11, n + 1000, 2], dtype=np.int32)
    gk2, gv2, gb2 = _merge_gpu(inp["hist_k"], inp["hist_v"], bad_off, bad_mem, "bf16")
    hk = inp["hist_k"].astype(np.float64)
    for got, want in ((gk2[0], hk[5] / 3), (gk2[1], 0 * hk[0]), (gk2[2], hk[9]), (gk2[3], (hk[11] + hk[2]) / 3)):
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)
    assert gb2[1] == -np.inf and gb2[0] == pytest.approx(np.log(3.0), abs=1e-6)


def _merged_case(inp):
    """GPU merge of the history, then the biased attention; the merged cache replaces the history."""
    torch = torch_mod()
    off, mem = inp["hist_groups"]
    G = off.size - 1
    H, dh = inp["hist_k"].shape[1], inp["hist_k"].shape[2]
    import kv_cache_attention_split_amd as ispa
    dev = {k: to_dev(inp[k], inp["dtype"]) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    mk = torch.empty((G, H, dh), dtype=tdt, device="cuda")
    mv = torch.empty((G, H, dh), dtype=tdt, device="cuda")
    mb = torch.empty((G,), dtype=torch.float32, device="cuda")
    ispa.ispa_kv_merge(dev["hist_k"], dev["hist_v"], torch.from_numpy(off).cuda(), torch.from_numpy(mem).cuda(),
                       mk, mv, mb)
    n_q = inp["q"].shape[0]
    out = empty_outputs(n_q, H, dh, inp["dtype"])
    ispa.ispa_attn_dual_biased(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"], mk, mv,
                               float(inp["scale"]), out["a_loc"], out["a_full"], out["lse_loc"],
                               out["lse_hist"], out["lse_full"], hist_bias=mb)
    torch.cuda.synchronize()
    return dev, out, G


def test_lemma_on_gpu_merged_history_matches_original():
    inp = inputs.static_history_case(11, n_heads=2, head_dim=128, n_q=260, n_sink=64, n_cur=200, n_frames=6,
                                     frame_tokens=150, static_frac=0.5)
    _log("case: merged history (6 frames x 150 tokens, half static) vs the original, 2 x 128")
    ref = oatt.dual_stream(inp)                     # the original, unmerged cache
    dev, merged, G = _merged_case(inp)
    assert G == 75 + 6 * 75
    rep = check_attention(merged, ref, "bf16")
    _, orig = run_attn(inp, dev=dev)
    check_attention(orig, ref, "bf16")
    _log(f"   merged vs oracle of the original: {rep}")


def test_lemma_wan_shape_sampled_rows():
    # 12 heads x 128, one 4680-query chunk, sink and current chunk of 4680 keys each, a 6-frame
    # history (9360 keys) whose half is static: merged to 4680 + 780 = 5460 rows
    inp = inputs.static_history_case(12, n_heads=12, head_dim=128, n_q=4680, n_sink=4680, n_cur=4680,
                                     n_frames=6, frame_tokens=1560, static_frac=0.5)
    _log("case: Wan-shaped merged history, 12 x 128, 4680 queries, sampled rows")
    dev, merged, G = _merged_case(inp)
    assert G == 780 + 6 * 780
    rows = np.random.default_rng(1).choice(4680, size=48, replace=False)
    rows.sort()
    ref = oatt.dual_stream(inp, rows=rows)
    rep = check_attention(merged, ref, "bf16", rows=rows)
    _log(f"   {rep}")
