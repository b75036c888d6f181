"""GPU parity of the L-Layer steady state (weight update, output projection) against the oracle.

Gates: the bf16 weights W + dW are bit-exact (the fp32 sum and its rounding are the same decision on
both sides); the projection y = A W^T is within half a bf16 unit of the exact result plus the fp32
accumulation error, |y - y_ref| <= 2^-8 |y_ref| + 2^-16 sum_k |a_k w_k|.
"""
import numpy as np
import pytest

from oracle import steady as ost

from gpu_helpers import to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _bits_dev(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _bf16_values(rng, shape, scale=1.0):
    x = (scale * rng.standard_normal(shape)).astype(np.float32)
    return ost.bf16_bits_to_f64(ost.round_to_bf16_bits(x)).astype(np.float32)


@pytest.mark.parametrize("d_in,d_out,linear", [(70, 50, False), (70, 50, True), (1536, 1536, False),
                                               (1536, 1536, True), (1, 8, False)])
def test_apply_delta_bit_exact(d_in, d_out, linear):
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    _log(f"case: apply_delta d_in={d_in} d_out={d_out} linear={linear}")
    rng = np.random.default_rng(d_in * 7 + d_out + int(linear))
    shape = (d_out, d_in) if linear else (d_in, d_out)
    w = (rng.standard_normal(shape) / np.sqrt(d_in)).astype(np.float32)
    dw = (1e-2 * rng.standard_normal(shape) / np.sqrt(d_in)).astype(np.float32)
    out = torch.full((d_out, d_in), float("nan"), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_apply_delta(torch.from_numpy(w).cuda(), torch.from_numpy(dw).cuda(), out, w_is_linear_weight=linear)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    want = ost.apply_delta(w, dw, w_is_linear_weight=linear)
    assert np.array_equal(got, want)


def _check_projection(a, wl, y):
    ref = ost.project(a, wl)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * (np.abs(a.astype(np.float64)) @ np.abs(wl.astype(np.float64)).T)
    err = np.abs(y - ref)
    assert np.all(err <= bound), f"max excess {float(np.max(err - bound))}"
    return float(np.max(err))


@pytest.mark.parametrize("n,d_in,d_out,pad", [(300, 64, 200, 0), (1, 32, 8, 0), (517, 192, 136, 24),
                                              (129, 96, 264, 8), (4680, 1536, 1536, 0)])
def test_projection_full_compare(n, d_in, d_out, pad):
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    _log(f"case: project n={n} d_in={d_in} d_out={d_out} pad={pad}")
    rng = np.random.default_rng(n + d_in + d_out)
    a = _bf16_values(rng, (n, d_in))
    wl = _bf16_values(rng, (d_out, d_in), scale=1.0 / np.sqrt(d_in))
    a_store = torch.zeros((n, d_in + pad), dtype=torch.bfloat16, device="cuda")
    a_store[:, :d_in] = to_dev(a, "bf16")
    y_store = torch.full((n, d_out + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_project(a_store[:, :d_in], to_dev(wl, "bf16"), y_store[:, :d_out])
    torch.cuda.synchronize()
    y = to_host64(y_store[:, :d_out])
    err = _check_projection(a, wl, y)
    if pad:
        assert torch.isnan(y_store[:, d_out:]).all(), "wrote outside the output rows"
    _log(f"   max |y - y_ref| = {err:.3g}")


def test_projection_empty_is_noop():
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    a = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_project(a, w, y)
    torch.cuda.synchronize()


def test_l_layer_chain_local_attention_then_updated_projection():
    # an L-Layer after the warmup: local-only attention (empty history, no A_full), weights updated by
    # the absorb delta, projection; compared with the oracle on the GPU's own A_loc and dW
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    from gpu_helpers import run_attn
    torch = torch_mod()
    _log("case: L-Layer chain (local attention, apply_delta, project), 4 heads x 64, 300 queries")
    inp = inputs.attention_case(31, n_heads=4, head_dim=64, n_q=300, n_sink=64, n_cur=300, n_hist=0,
                                dtype="bf16")
    _, out = run_attn(inp, want_full=False)
    a_loc = to_host64(out["a_loc"]).astype(np.float32)        # exact bf16 values
    d = a_loc.shape[1]
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    dw = (3e-2 * rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    w_new = torch.empty((d, d), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_apply_delta(torch.from_numpy(w).cuda(), torch.from_numpy(dw).cuda(), w_new)
    y = torch.empty((a_loc.shape[0], d), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_project(out["a_loc"], w_new, y)
    torch.cuda.synchronize()
    wl_ref = ost.bf16_bits_to_f64(ost.apply_delta(w, dw)).astype(np.float32)
    assert np.array_equal(w_new.cpu().view(torch.int16).numpy().view(np.uint16), ost.apply_delta(w, dw))
    _check_projection(a_loc, wl_ref, to_host64(y))
