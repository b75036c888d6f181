"""The allocation-free future-score entry point against the workspace one, through the C ABI.

ispa_future_scores_noalloc runs the same kernels as ispa_future_scores with the library's per-GPU
scratch array in place of the caller's workspace (Future Forcing summary page, "Componenti
Algorithmiche", module 1: keys scored by the mean attention weight of proxy queries). Two calls in a row
on one GPU, the second smaller than the first, must each give the workspace entry point's scores bit for
bit: the array keeps the first call's contents, and the second call must not read any of them.
"""
import numpy as np
import pytest

import ispa_inputs as inputs

from gpu_helpers import to_dev, torch_mod

pytestmark = pytest.mark.gpu


def _case(seed, H, n_p, n_sink, n_cur, n_hist):
    inp = inputs.attention_case(seed, H, 128, n_p, n_sink, n_cur, n_hist, dtype="bf16", rho=0.95)
    return {k: to_dev(inp[k], "bf16") for k in ("q", "sink_k", "cur_k", "hist_k")}, inp["scale"]


def _both(dev, scale, lam=0.3):
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    H = dev["q"].shape[1]
    n = sum(int(dev[k].shape[0]) for k in ("sink_k", "cur_k", "hist_k"))
    hist_tok = torch.linspace(0.0, 1.0, n, device="cuda", dtype=torch.float32)
    out = {}
    for name in ("workspace", "noalloc"):
        scores = torch.full((H, n), float("nan"), dtype=torch.float32, device="cuda")
        tok = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        if name == "workspace":
            ws = torch.empty(ispa.ispa_future_scores_workspace(H, dev["q"].shape[0]), dtype=torch.uint8,
                             device="cuda")
            ispa.ispa_future_scores(dev["q"], dev["sink_k"], dev["cur_k"], dev["hist_k"], scale, scores, ws, lam,
                                    hist_tok, tok)
        else:
            ispa.ispa_future_scores_noalloc(dev["q"], dev["sink_k"], dev["cur_k"], dev["hist_k"], scale, scores,
                                            lam, hist_tok, tok)
        torch.cuda.synchronize()
        out[name] = (scores, tok)
    return out


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    torch = torch_mod()
    # first: 12 heads x 1560 proxies (key ranges split three ways) over 3 frames of sink/current and 6 of
    # history; second: 2 heads x 300 proxies (16 key splits) over a few hundred keys
    cases = [(1, 12, 1560, 1560, 1560, 9360), (2, 2, 300, 70, 100, 333)]
    for seed, H, n_p, n_s, n_c, n_h in cases:
        print(f"case: future scores noalloc vs workspace, H={H} proxies={n_p} keys={n_s}/{n_c}/{n_h}", flush=True)
        dev, scale = _case(seed, H, n_p, n_s, n_c, n_h)
        out = _both(dev, scale)
        s_ws, t_ws = out["workspace"]
        s_na, t_na = out["noalloc"]
        assert torch.isfinite(s_na).all() and torch.isfinite(t_na).all()
        assert torch.equal(s_ws, s_na), float((s_ws - s_na).abs().max())
        assert torch.equal(t_ws, t_na)
        sums = s_na.double().sum(dim=1).cpu().numpy()
        assert np.all(np.abs(sums - 1.0) <= 1e-4), sums   # each head's scores are weights summing to 1


def test_noalloc_rejects_calls_beyond_its_scratch():
    import kv_cache_attention_split_amd as ispa
    from kv_cache_attention_split_amd import _abi
    torch = torch_mod()
    H, n_p = 64, 40000      # needs more than the library's 16 MiB array
    assert ispa.ispa_future_scores_workspace(H, n_p) > _abi.ISPA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((n_p, H, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((8, H, 128), dtype=torch.bfloat16, device="cuda")
    scores = torch.zeros((H, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(ispa.IspaError) as e:
        ispa.ispa_future_scores_noalloc(q, None, k, None, 0.088, scores)
    assert e.value.status == _abi.ISPA_E_WORKSPACE
