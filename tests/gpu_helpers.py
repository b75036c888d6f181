"""Helpers for the GPU parity tests: host<->device conversion of the seeded inputs and comparisons."""
from __future__ import annotations

import numpy as np

import ispa_inputs as inputs


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray, dtype: str):
    """Exact float32 values -> device tensor of the workload dtype ("bf16" or "f32")."""
    torch = torch_mod()
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        bits = inputs.bf16_bits(x)
        assert np.array_equal(inputs.bf16_bits_to_f32(bits), x), "input is not exactly bf16"
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(x)
    return t.to("cuda")


def to_host64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def empty_outputs(n_q: int, H: int, dh: int, dtype: str, want_full: bool = True):
    torch = torch_mod()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {
        "a_loc": torch.full((n_q, H * dh), float("nan"), dtype=tdt, device="cuda"),
        "a_full": torch.full((n_q, H * dh), float("nan"), dtype=tdt, device="cuda") if want_full else None,
        "lse_loc": torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda"),
        "lse_hist": torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda") if want_full else None,
        "lse_full": torch.full((H, n_q), float("nan"), dtype=torch.float32, device="cuda") if want_full else None,
    }
    return out


def run_attn(inp, want_full: bool = True, dev=None, stream=None):
    """Upload one attention case and run ispa_attn_dual. Returns (device inputs, device outputs)."""
    import kv_cache_attention_split_amd as ispa
    dt = inp["dtype"]
    if dev is None:
        dev = {k: to_dev(inp[k], dt) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    n_q, H, dh = inp["q"].shape
    out = empty_outputs(n_q, H, dh, dt, want_full)
    ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"],
                        dev["hist_k"], dev["hist_v"], float(inp["scale"]), out["a_loc"], out["a_full"],
                        out["lse_loc"], out["lse_hist"], out["lse_full"], stream=stream)
    torch_mod().cuda.synchronize()
    return dev, out


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


# Tolerances for the attention outputs on identical inputs. bf16: A max-abs 1e-2 and LSE 1e-3 abs (the
# stated bounds), plus a relative-Frobenius guard of 1e-2 (outputs of size ~n_keys^-1/2 make the
# absolute bound alone weak). Storing A in bf16 rounds each element by up to 2^-9 |A| and the bf16
# probabilities add about as much again, so where outputs are O(1) (a handful of keys) the absolute
# bound widens by 2^-7 |A|: |err| <= 1e-2 + 2^-7 |A_ref|, the same as 1e-2 at workload sizes.
ATT_BF16 = {"a_max_abs": 1e-2, "a_rel": 2.0 ** -7, "a_rel_fro": 1e-2, "lse_abs": 1e-3}
ATT_F32 = {"a_max_abs": 1e-5, "a_rel": 1e-5, "a_rel_fro": 1e-5, "lse_abs": 1e-5}


def check_attention(out, ref, dtype: str, rows=None, heads=None):
    tol = ATT_BF16 if dtype == "bf16" else ATT_F32
    pairs = (("a_loc", "A_loc"), ("a_full", "A_full"))
    report = {}
    for mine, theirs in pairs:
        if out[mine] is None:
            continue
        got = to_host64(out[mine])
        if rows is not None:
            got = got[rows]
        want = ref[theirs]
        assert np.all(np.isfinite(got)), f"{mine} has non-finite values"
        report[mine] = (max_abs(got, want), rel_fro(got, want))
        excess = np.abs(got - want) - (tol["a_max_abs"] + tol["a_rel"] * np.abs(want))
        assert np.all(excess <= 0), (mine, report[mine], float(excess.max()))
        assert report[mine][1] <= tol["a_rel_fro"], (mine, report[mine])
    for mine, theirs in (("lse_loc", "lse_loc"), ("lse_hist", "lse_hist"), ("lse_full", "lse_full")):
        if out[mine] is None:
            continue
        got = to_host64(out[mine])
        if rows is not None:
            got = got[:, rows]
        want = ref[theirs]
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(got), fin), f"{mine}: finiteness differs"
        assert np.all(got[~fin] == want[~fin]), f"{mine}: infinities differ"
        err = max_abs(got[fin], want[fin]) if fin.any() else 0.0
        report[mine] = err
        assert err <= tol["lse_abs"], (mine, err)
    return report


def admissible_selection(sel, eps_ref, k: int, tol: float) -> None:
    """Assert that `sel` is a selection the layer-ranking rule admits when errors are known to within
    a relative `tol`: k distinct layers, and no selected layer's oracle error exceeds an unselected
    layer's by more than the tolerance allows, max_{i in sel} eps_i <= (1 + tol)/(1 - tol) * min_{j not
    in sel} eps_j. When the k-th and (k+1)-th errors are further apart than that, the only admissible
    set is the oracle's own."""
    eps_ref = np.asarray(eps_ref, dtype=np.float64)
    sel = [int(i) for i in sel]
    assert len(sel) == k and len(set(sel)) == k, sel
    rest = [j for j in range(len(eps_ref)) if j not in set(sel)]
    if not rest or not sel:
        return
    r = (1.0 + tol) / (1.0 - tol)
    worst_in = float(eps_ref[sel].max())
    best_out = float(eps_ref[rest].min())
    assert worst_in <= r * best_out, (sel, worst_in, best_out)


def bf16_p_sigma(inp, rows=None):
    """Spread of each output element [n_q or len(rows), H*d_h] that rounding the probabilities to bf16
    (the value product's operand) causes: independent errors uniform over half a bf16 spacing, 2^-8
    relative, so std p 2^-8 / sqrt(3); probabilities from exact float64 scores against the true maximum
    (the device's running maximum never exceeds it). Returns {"A_loc": ..., "A_full": ...}."""
    q = np.asarray(inp["q"], np.float64)
    if rows is not None:
        q = q[rows]
    scale = float(inp["scale"])
    segs = {"A_loc": ("sink", "cur"), "A_full": ("sink", "cur", "hist")}
    out = {}
    n_q, H, dh = q.shape
    for name, names in segs.items():
        k = np.concatenate([np.asarray(inp[n + "_k"], np.float64) for n in names])
        v = np.concatenate([np.asarray(inp[n + "_v"], np.float64) for n in names])
        sig = np.zeros((n_q, H * dh))
        for h in range(H):
            sc = scale * (q[:, h, :] @ k[:, h, :].T)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            L = p.sum(axis=1, keepdims=True)
            err = p * 2.0 ** -8 / np.sqrt(3.0)
            sig[:, h * dh:(h + 1) * dh] = np.sqrt((err / L) ** 2 @ (v[:, h, :] ** 2))
        out[name] = sig
    return out


def check_attention_tight(out, ref, sig, rows=None, sigmas=6.0):
    """bf16 rows against the oracle within the arithmetic's own bound: `sigmas` x the bf16 probability-
    rounding spread plus the bf16 rounding of the stored row (2^-9 |A|, doubled) plus 1e-6. Returns the
    largest error in units of sigma."""
    worst = {}
    for mine, theirs in (("a_loc", "A_loc"), ("a_full", "A_full")):
        if out[mine] is None:
            continue
        got = to_host64(out[mine])
        if rows is not None:
            got = got[rows]
        want, sg = ref[theirs], sig[theirs]
        err = np.abs(got - want)
        excess = err - (sigmas * sg + 2.0 ** -8 * np.abs(want) + 1e-6)
        assert np.all(excess <= 0), (mine, float(excess.max()), float((err / (sg + 1e-30)).max()))
        worst[mine] = float(((err - 2.0 ** -8 * np.abs(want)).clip(0) / (sg + 1e-30)).max())
    return worst
