"""GPU parity of ispa_attn_dual against the fp64 oracle (same seeded inputs).

Small cases are compared element by element over every output; workload-size cases (1.3B chunk 4,
14B chunk 4, the 60-frame-history rollout) are compared on sampled query rows, which the oracle
evaluates one by one, plus properties that hold at any size.
"""
import math

import numpy as np
import pytest

import ispa_inputs as inputs
from oracle import attention as oatt

from gpu_helpers import (bf16_p_sigma, check_attention, check_attention_tight, run_attn, to_dev, to_host64, empty_outputs, torch_mod,
                         max_abs, rel_fro)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def test_workload1_fp32_full_compare():
    inp = inputs.attention_inputs(1)
    _log("case: workload 1 (fp32, 2x64, 128 q, 64/128/512 keys)")
    _, out = run_attn(inp)
    ref = oatt.dual_stream(inp)
    rep = check_attention(out, ref, "f32")
    _log(f"  {rep}")


@pytest.mark.parametrize("case", [
    # seed, H, dh, n_q, sink, cur, hist  (several tiles, ragged tails everywhere)
    (1, 2, 128, 300, 70, 100, 333),
    (2, 3, 64, 130, 0, 64, 65),
    (3, 1, 128, 129, 1, 0, 1),
    (4, 2, 128, 64, 5, 7, 0),
    (5, 2, 64, 257, 200, 300, 700),
])
def test_bf16_small_full_compare(case):
    seed, H, dh, n_q, ns, nc, nh = case
    _log(f"case: bf16 seed={seed} H={H} dh={dh} n_q={n_q} sink={ns} cur={nc} hist={nh}")
    inp = inputs.attention_case(seed, H, dh, n_q, ns, nc, nh, dtype="bf16", rho=0.95)
    _, out = run_attn(inp)
    ref = oatt.dual_stream(inp)
    rep = check_attention(out, ref, "bf16")
    _log(f"  {rep}")


def score_jump_case(seed: int):
    """Keys of a few 64-key tiles scaled up (x2, x3, x4, x6), so that the running maximum of many rows
    jumps by a few to many log2 units in the middle of the local and the history keys: the softmax
    raises its reference, rescales the accumulator, or recomputes a tile without raising it."""
    inp = inputs.attention_case(seed, 2, 128, 260, 16, 200, 400, dtype="bf16")
    hk = inp["hist_k"].copy()
    for t, f in ((1, 2.0), (3, 3.0), (5, 6.0)):
        hk[64 * t:64 * (t + 1)] *= f
    ck = inp["cur_k"].copy()
    ck[100:164] *= 4.0
    inp["hist_k"], inp["cur_k"] = inputs.round_bf16(hk), inputs.round_bf16(ck)
    return inp


def test_bf16_score_jumps_mid_stream():
    inp = score_jump_case(11)
    _log("case: bf16 2 x 128, 260 queries, 16/200/400 keys with scaled key tiles (maximum jumps)")
    _, out = run_attn(inp)
    rep = check_attention(out, oatt.dual_stream(inp), "bf16")
    _log(f"  {rep}")


def test_fp32_head128_and_ragged():
    inp = inputs.attention_case(7, 2, 128, 150, 33, 40, 97, dtype="f32")
    _log("case: fp32 H=2 dh=128 n_q=150 33/40/97")
    _, out = run_attn(inp)
    check_attention(out, oatt.dual_stream(inp), "f32")


def test_empty_history_is_bitwise_local():
    inp = inputs.attention_case(8, 2, 128, 200, 64, 100, 0, dtype="bf16")
    _log("case: empty history")
    _, out = run_attn(inp)
    torch = torch_mod()
    assert torch.equal(out["a_full"], out["a_loc"])
    assert torch.equal(out["lse_full"], out["lse_loc"])
    assert bool(torch.all(torch.isneginf(out["lse_hist"])))
    check_attention(out, oatt.dual_stream(inp), "bf16")


def test_local_only_call_matches_dual_local():
    """a_full = NULL computes the local branch alone; it equals the dual call's A_loc bitwise."""
    inp = inputs.attention_case(9, 2, 128, 190, 64, 130, 300, dtype="bf16")
    _log("case: local-only vs dual")
    dev, out = run_attn(inp)
    _, out_l = run_attn(inp, want_full=False, dev=dev)
    torch = torch_mod()
    assert torch.equal(out_l["a_loc"], out["a_loc"])
    assert torch.equal(out_l["lse_loc"], out["lse_loc"])


def test_zero_queries_uniform_weights():
    """P-3 on the device: Q = 0 gives uniform weights, lse = log(n) and A = mean of V."""
    inp = inputs.attention_case(10, 2, 128, 96, 100, 200, 1000, dtype="bf16")
    inp["q"] = np.zeros_like(inp["q"])
    _log("case: Q = 0")
    _, out = run_attn(inp)
    n_loc, n_all = 300, 1300
    lse_loc = to_host64(out["lse_loc"])
    lse_full = to_host64(out["lse_full"])
    lse_hist = to_host64(out["lse_hist"])
    assert np.max(np.abs(lse_loc - math.log(n_loc))) <= 1e-6 * math.log(n_loc)
    assert np.max(np.abs(lse_full - math.log(n_all))) <= 1e-6 * math.log(n_all)
    assert np.max(np.abs(lse_hist - math.log(1000))) <= 1e-6 * math.log(1000)
    ref = oatt.dual_stream(inp)
    check_attention(out, ref, "bf16")


def _scores_against(inp, kstar):
    """tau q . k* for every (head, query) in float64 on the exact input values: [H, n_q]."""
    q = inp["q"].astype(np.float64)
    return float(inp["scale"]) * np.einsum("qhd,hd->hq", q, kstar.astype(np.float64))


@pytest.mark.parametrize("dh", [64, 128])
def test_equal_keys_closed_form(dh):
    """P-3 on the device: when every key equals one k*, all weights are equal, so lse_X = tau q.k* +
    log n_X and A_X is the mean of segment X's values (closed forms, no oracle code)."""
    n_q, n_s, n_c, n_h = 160, 70, 90, 300
    inp = inputs.attention_case(21, 2, dh, n_q, n_s, n_c, n_h, dtype="bf16")
    kstar = inp["cur_k"][0].copy()
    for name in ("sink_k", "cur_k", "hist_k"):
        inp[name][:] = kstar[None]
    _log(f"case: all keys equal, d_h={dh}")
    _, out = run_attn(inp)
    s = _scores_against(inp, kstar)
    for name, n in (("lse_loc", n_s + n_c), ("lse_hist", n_h), ("lse_full", n_s + n_c + n_h)):
        want = s + math.log(n)
        got = to_host64(out[name])
        err = float(np.max(np.abs(got - want) / np.maximum(np.abs(want), 1.0)))
        assert err <= 1e-6, (name, err)
    v_loc = np.concatenate([inp["sink_v"], inp["cur_v"]]).astype(np.float64).mean(axis=0)
    v_all = np.concatenate([inp["sink_v"], inp["cur_v"], inp["hist_v"]]).astype(np.float64).mean(axis=0)
    for name, m in (("a_loc", v_loc), ("a_full", v_all)):
        got = to_host64(out[name]).reshape(n_q, 2, dh)
        err = float(np.max(np.abs(got - m[None])))
        assert err <= 2.0 ** -8 * float(np.max(np.abs(m))) + 1e-6, (name, err)


def test_single_key_gives_its_value():
    """P-3 on the device: one local key and no history give A_loc = A_full = v of that key exactly and
    lse_loc = lse_full = tau q.k, lse_hist = -inf."""
    torch = torch_mod()
    inp = inputs.attention_case(22, 2, 128, 100, 0, 1, 0, dtype="bf16")
    _, out = run_attn(inp)
    v = inp["cur_v"][0].astype(np.float64)
    got = to_host64(out["a_loc"]).reshape(100, 2, 128)
    assert np.array_equal(got, np.broadcast_to(v, got.shape))
    assert torch.equal(out["a_full"], out["a_loc"])
    want = _scores_against(inp, inp["cur_k"][0])
    for name in ("lse_loc", "lse_full"):
        got = to_host64(out[name])
        assert float(np.max(np.abs(got - want) / np.maximum(np.abs(want), 1.0))) <= 1e-6, name
    assert np.all(np.isneginf(to_host64(out["lse_hist"])))


def test_constant_values_give_constant_output():
    """P-3 on the device: when every value row equals one c, A_loc = A_full = c whatever the weights
    (up to the bf16 rounding of the probabilities and of the output)."""
    n_q, n_s, n_c, n_h = 130, 40, 90, 200
    inp = inputs.attention_case(23, 2, 128, n_q, n_s, n_c, n_h, dtype="bf16")
    c = inp["cur_v"][0].copy()
    for name in ("sink_v", "cur_v", "hist_v"):
        inp[name][:] = c[None]
    _, out = run_attn(inp)
    c64 = c.astype(np.float64)
    for name in ("a_loc", "a_full"):
        got = to_host64(out[name]).reshape(n_q, 2, 128)
        err = float(np.max(np.abs(got - c64[None]) / np.maximum(np.abs(c64[None]), 1e-3)))
        assert err <= 2.0 ** -7, (name, err)
    ref = oatt.dual_stream(inp)
    check_attention(out, ref, "bf16")


def test_deterministic_repeat():
    inp = inputs.attention_case(11, 2, 128, 200, 64, 100, 250, dtype="bf16")
    dev, out1 = run_attn(inp)
    _, out2 = run_attn(inp, dev=dev)
    torch = torch_mod()
    for k in ("a_loc", "a_full", "lse_loc", "lse_hist", "lse_full"):
        assert torch.equal(out1[k], out2[k]), k


def test_strided_rows():
    """Token rows with a stride larger than H*d_h (a view into a wider buffer)."""
    torch = torch_mod()
    inp = inputs.attention_case(12, 2, 64, 100, 30, 60, 90, dtype="bf16")
    dev = {}
    for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v"):
        x = to_dev(inp[k], "bf16")
        n = x.shape[0]
        wide = torch.zeros((n, 3, 64), dtype=x.dtype, device="cuda")
        wide[:, 1:3] = x
        dev[k] = wide[:, 1:3]
    _log("case: strided rows")
    _, out = run_attn(inp, dev=dev)
    check_attention(out, oatt.dual_stream(inp), "bf16")


def _sampled(cfg, chunk=0, n_rows=48, seed=0, heads=None):
    inp = inputs.attention_inputs(cfg, 0, chunk)
    rng = np.random.default_rng(seed)
    n_q = inp["q"].shape[0]
    rows = np.unique(np.concatenate([rng.choice(n_q, n_rows, replace=False), [0, n_q - 1]]))
    return inp, rows


@pytest.mark.parametrize("cfg", [2, 5])
def test_workload_sampled_rows(cfg):
    inp, rows = _sampled(cfg)
    s = inputs.CONFIGS[cfg].segment_sizes()
    _log(f"case: workload {cfg} sampled rows ({len(rows)}) {s}")
    _, out = run_attn(inp)
    ref = oatt.dual_stream(inp, rows=rows)
    rep = check_attention(out, ref, "bf16", rows=rows)
    _log(f"  {rep}")


def test_workload4_chunk4_sampled_rows():
    inp, rows = _sampled(4, chunk=3, n_rows=24)
    _log("case: workload 4 chunk 4 (40 heads) sampled rows")
    _, out = run_attn(inp)
    ref = oatt.dual_stream(inp, rows=rows)
    rep = check_attention(out, ref, "bf16", rows=rows)
    _log(f"  {rep}")


def test_workload5_merge_equals_single_pass():
    """The dual call's A_full/lse_full equal a single pass with all keys in the local run, and
    lse_full = logaddexp(lse_loc, lse_hist) on the device outputs."""
    torch = torch_mod()
    inp = inputs.attention_inputs(5)
    _log("case: workload 5 merge vs single pass")
    dev, out = run_attn(inp)
    one = dict(inp)
    one["cur_k"] = np.concatenate([inp["cur_k"], inp["hist_k"]])
    one["cur_v"] = np.concatenate([inp["cur_v"], inp["hist_v"]])
    one["hist_k"] = inp["hist_k"][:0]
    one["hist_v"] = inp["hist_v"][:0]
    dev1 = dict(dev)
    dev1["cur_k"] = torch.cat([dev["cur_k"], dev["hist_k"]])
    dev1["cur_v"] = torch.cat([dev["cur_v"], dev["hist_v"]])
    dev1["hist_k"] = dev["hist_k"][:0]
    dev1["hist_v"] = dev["hist_v"][:0]
    _, single = run_attn(one, dev=dev1)
    a_dual = to_host64(out["a_full"])
    a_single = to_host64(single["a_loc"])
    assert max_abs(a_dual, a_single) <= 2e-3
    assert rel_fro(a_dual, a_single) <= 5e-3
    assert max_abs(to_host64(out["lse_full"]), to_host64(single["lse_loc"])) <= 1e-4
    lse = np.logaddexp(to_host64(out["lse_loc"]), to_host64(out["lse_hist"]))
    assert max_abs(lse, to_host64(out["lse_full"])) <= 1e-4


# ---- balanced schedule (ispa_attn_dual_balanced) ----------------------------------------------------
def run_attn_balanced(inp, want_full=True):
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    dt = inp["dtype"]
    dev = {k: to_dev(inp[k], dt) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    n_q, H, dh = inp["q"].shape
    out = empty_outputs(n_q, H, dh, dt, want_full)
    n_loc = inp["sink_k"].shape[0] + inp["cur_k"].shape[0]
    n_hist = inp["hist_k"].shape[0] if want_full else 0
    need = ispa.ispa_attn_dual_balanced_workspace(dev["q"], n_loc, n_hist)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ispa.ispa_attn_dual_balanced(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"], dev["hist_k"],
                                 dev["hist_v"], float(inp["scale"]), out["a_loc"], out["a_full"], out["lse_loc"],
                                 out["lse_hist"], out["lse_full"], ws=ws)
    torch.cuda.synchronize()
    return need, out


def _same_outputs(x, y):
    torch = torch_mod()
    return all((x[k] is None and y[k] is None) or torch.equal(x[k], y[k]) for k in x)


@pytest.mark.parametrize("cfg,chunk", [(2, 0), (3, 0)])
def test_balanced_workload_rows(cfg, chunk):
    """12 heads x 19 query tiles leave 28 of 256 compute units idle: the balanced schedule cuts units
    between workgroups (config 2: local and history keys; config 3 chunk 1: local keys only, so the
    local branch itself is merged). Sampled rows of all heads against the oracle, the plain call within
    the same bounds, and the call repeated bit for bit."""
    inp, rows = _sampled(cfg, chunk=chunk, n_rows=40, seed=7)
    _log(f"case: balanced schedule, workload {cfg} chunk {chunk + 1}, sampled rows ({len(rows)})")
    need, out = run_attn_balanced(inp)
    assert need > 0, "expected the balanced schedule at 12 heads"
    ref = oatt.dual_stream(inp, rows=rows)
    rep = check_attention(out, ref, "bf16", rows=rows)
    sig = bf16_p_sigma(inp, rows=rows)
    _log(f"  {rep}; worst element in bf16-rounding sigmas: balanced {check_attention_tight(out, ref, sig, rows)}")
    _, out2 = run_attn_balanced(inp)
    assert _same_outputs(out, out2), "balanced schedule not repeatable"
    # the plain call meets the same bound, and the two differ by two independent roundings of the
    # probabilities (each against its own running maximum): sqrt(2) sigma, and the LSEs by fp32 sums
    _, plain = run_attn(inp)
    _log(f"  plain: {check_attention_tight(plain, ref, sig, rows)}")
    for k, name in (("a_loc", "A_loc"), ("a_full", "A_full")):
        x, y = to_host64(out[k])[rows], to_host64(plain[k])[rows]
        excess = np.abs(x - y) - (6.0 * np.sqrt(2.0) * sig[name] + 2.0 ** -7 * np.abs(y) + 2e-6)
        assert np.all(excess <= 0), (k, float(excess.max()))
    for k in ("lse_loc", "lse_hist", "lse_full"):
        x, y = to_host64(out[k]), to_host64(plain[k])
        fin = np.isfinite(y)
        assert np.array_equal(np.isfinite(x), fin)
        assert np.all(np.abs(x[fin] - y[fin]) <= 1e-5), (k, float(np.abs(x[fin] - y[fin]).max()))


def _tile_rows(n_q, seed):
    """Three query rows of every 256-query tile (its first, its last and one between): every unit of
    every head is checked."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, n_q, 256):
        t1 = min(n_q, t0 + 256)
        rows += [t0, t1 - 1, int(rng.integers(t0, t1))]
    return np.unique(np.array(rows))


def _balanced_against_oracle_and_plain(inp, rows, want_full=True):
    need, out = run_attn_balanced(inp, want_full=want_full)
    assert need > 0, "expected the balanced schedule"
    ref = oatt.dual_stream(inp, rows=rows)
    rep = check_attention(out, ref, "bf16", rows=rows)
    sig = bf16_p_sigma(inp, rows=rows)
    _log(f"  {rep}; worst element in bf16-rounding sigmas: {check_attention_tight(out, ref, sig, rows)}")
    _, out2 = run_attn_balanced(inp, want_full=want_full)
    assert _same_outputs(out, out2), "balanced schedule not repeatable"
    if want_full:
        _, plain = run_attn(inp)
        for k in ("lse_loc", "lse_hist", "lse_full"):
            x, y = to_host64(out[k]), to_host64(plain[k])
            fin = np.isfinite(y)
            assert np.array_equal(np.isfinite(x), fin), k
            assert np.all(np.abs(x[fin] - y[fin]) <= 1e-5), (k, float(np.abs(x[fin] - y[fin]).max()))
    return out


def test_balanced_cut_inside_local_keys():
    """12 heads x 15 query tiles (180 units, the last tile ragged): each XCD's main workgroups stop at
    R = 45 or 47 of 58 key tiles, inside the local keys (48 tiles), so A_loc is merged too, and the
    spare workgroups' ranges cut units' remaining tiles both at range boundaries and at the local end."""
    inp = inputs.attention_case(23, 12, 128, 3800, 40, 3000, 600, dtype="bf16", rho=0.95)
    _log("case: balanced schedule, 12 x 128, 3800 queries, 40/3000/600 keys (cuts inside the local keys)")
    _balanced_against_oracle_and_plain(inp, _tile_rows(3800, 1))


def test_balanced_main_piece_ends_at_local_end():
    """8 heads x 16 query tiles (128 units: 16 per XCD, as many spare workgroups as main ones, so the
    spare ranges are whole units' remaining tiles) with 26 local and 14 history key tiles: R = 16 x 40 /
    32 + 6 = 26, the main piece ends exactly at the local end and writes A_loc itself."""
    inp = inputs.attention_case(25, 8, 128, 4096, 32, 1632, 896, dtype="bf16")
    _log("case: balanced schedule, 8 x 128, 4096 queries, 32/1632/896 keys (main piece = local keys)")
    _balanced_against_oracle_and_plain(inp, _tile_rows(4096, 2))


def test_balanced_local_only_and_empty_history():
    inp = inputs.attention_case(24, 12, 128, 3800, 16, 5000, 700, dtype="bf16")
    _log("case: balanced schedule, local-only call and a call with an empty history (180 units)")
    rows = _tile_rows(3800, 3)
    _balanced_against_oracle_and_plain(inp, rows, want_full=False)
    inp0 = dict(inp, hist_k=inp["hist_k"][:0], hist_v=inp["hist_v"][:0])
    out0 = _balanced_against_oracle_and_plain(inp0, rows)
    torch = torch_mod()
    assert torch.equal(out0["a_full"], out0["a_loc"]) and torch.equal(out0["lse_full"], out0["lse_loc"])
    assert bool(torch.all(torch.isneginf(out0["lse_hist"])))


def test_balanced_plain_when_units_fill_the_gpu():
    """40 heads x 19 query tiles fill 256 compute units in three rounds, and 2 heads x 3 query tiles leave
    too few units to keep the lockstep per XCD: no workspace, the plain call."""
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    q = torch.empty((4680, 40, 128), dtype=torch.bfloat16, device="cuda")
    assert ispa.ispa_attn_dual_balanced_workspace(q, 9360, 9360) == 0
    q = torch.empty((600, 2, 128), dtype=torch.bfloat16, device="cuda")
    assert ispa.ispa_attn_dual_balanced_workspace(q, 3040, 9000) == 0
