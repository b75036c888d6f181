"""GPU parity of the future-query importance scores against the fp64 oracle (`oracle.future`).

Gates: every score within 1e-3 relative (+1e-7 absolute) of the oracle's mean softmax weight, each
head's scores summing to 1 within 1e-4, token and hybrid scores within the same bound; padding of
the score rows untouched.
"""
import numpy as np
import pytest

import ispa_inputs as inputs
from oracle import future as ofu

from gpu_helpers import to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _run(inp, pad=0, lam=None, hist_tok=None):
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    dev = {k: to_dev(inp[k], "bf16") for k in ("q", "sink_k", "cur_k", "hist_k")}
    H = inp["q"].shape[1]
    n = sum(inp[k].shape[0] for k in ("sink_k", "cur_k", "hist_k"))
    store = torch.full((H, n + pad), float("nan"), dtype=torch.float32, device="cuda")
    scores = store[:, :n]
    tok = None
    if lam is not None:
        tok = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ispa.ispa_future_scores(dev["q"], dev["sink_k"], dev["cur_k"], dev["hist_k"], float(inp["scale"]), scores,
                            lam=1.0 if lam is None else lam,
                            hist_token_score=None if hist_tok is None else torch.from_numpy(hist_tok).cuda(),
                            token_score=tok)
    torch.cuda.synchronize()
    if pad:
        assert torch.isnan(store[:, n:]).all(), "wrote into the score padding"
    return to_host64(scores), (None if tok is None else to_host64(tok))


def _check(got, ref):
    err = np.abs(got - ref)
    bound = 1e-3 * np.abs(ref) + 1e-7
    assert np.all(err <= bound), float(np.max(err / (np.abs(ref) + 1e-7)))
    assert np.all(np.abs(got.sum(axis=1) - 1.0) <= 1e-4)
    return float(np.max(err / (np.abs(ref) + 1e-7)))


@pytest.mark.parametrize("H,dh,n_p,ns,nc,nh,pad", [(2, 128, 100, 40, 70, 150, 0), (3, 128, 64, 0, 0, 333, 5),
                                                   (2, 64, 129, 17, 33, 300, 0), (1, 128, 1, 1, 0, 0, 0),
                                                   (2, 128, 300, 256, 256, 512, 3)])
def test_scores_vs_oracle(H, dh, n_p, ns, nc, nh, pad):
    _log(f"case: future scores H={H} d_h={dh} proxies={n_p} keys={ns}+{nc}+{nh} pad={pad}")
    inp = inputs.attention_case(90 + n_p, n_heads=H, head_dim=dh, n_q=n_p, n_sink=ns, n_cur=nc, n_hist=nh)
    got, _ = _run(inp, pad=pad)
    keys = np.concatenate([inp["sink_k"], inp["cur_k"], inp["hist_k"]], axis=0)
    ref = ofu.importance(inp["q"], keys, inp["scale"])
    rel = _check(got, ref)
    _log(f"   max rel err {rel:.2e}")


def test_token_and_hybrid_scores():
    inp = inputs.attention_case(95, n_heads=3, head_dim=128, n_q=90, n_sink=20, n_cur=50, n_hist=130)
    n = 200
    hist_tok = np.random.default_rng(2).random(n).astype(np.float32) / n
    got, tok = _run(inp, lam=0.3, hist_tok=hist_tok)
    keys = np.concatenate([inp["sink_k"], inp["cur_k"], inp["hist_k"]], axis=0)
    imp = ofu.importance(inp["q"], keys, inp["scale"])
    _check(got, imp)
    want = ofu.hybrid(ofu.token_scores(imp), hist_tok.astype(np.float64), 0.3)
    assert np.all(np.abs(tok - want) <= 1e-3 * np.abs(want) + 1e-7)
    # without a historical score the token score is lambda * future
    _, tok2 = _run(inp, lam=0.5)
    want2 = 0.5 * ofu.token_scores(imp)
    assert np.all(np.abs(tok2 - want2) <= 1e-3 * np.abs(want2) + 1e-7)


def test_wan_shape_three_heads():
    # 12 heads x 128, proxies of one future frame (1560), a cache of 4680 sink + 4680 current + 9360
    # history keys; the oracle on 3 of the 12 heads
    inp = inputs.attention_case(96, n_heads=12, head_dim=128, n_q=1560, n_sink=4680, n_cur=4680, n_hist=9360,
                                rho=0.95)
    _log("case: Wan-shaped future scores, 1560 proxies over 18720 keys, 12 x 128")
    got, _ = _run(inp)
    heads = [0, 5, 11]
    keys = np.concatenate([inp["sink_k"], inp["cur_k"], inp["hist_k"]], axis=0)
    ref = ofu.importance(inp["q"][:, heads], keys[:, heads], inp["scale"])
    rel = _check(got[heads], ref)
    assert np.all(np.abs(got.sum(axis=1) - 1.0) <= 1e-4)
    _log(f"   max rel err {rel:.2e}")
