#!/usr/bin/env python3
"""Benchmark of the ISPA hot path on one MI355X.

One step = one full ISPA warmup of a Wan-1.3B-shaped model (workload "wan1.3b-warmup"): for each of
the 4 chunks (4680 queries of a 3-frame chunk, history growing 0 -> 9 frames), the dual-stream
attention of each of the 30 layers (12 heads x 128) into that layer's rows of A_loc / A_full (each layer
keeps the rows of all its warmup chunks side by side, 18,720 x 1536 per output); after the last chunk
the warmup statistics of all 30 layers over all their rows in one batched call (the same sums as one
update per chunk, `--stats-per-chunk`, with a quarter of the statistics' read-modify-write traffic),
then one batched ridge solve of all layers (d = 1536, lambda = 1e-2) with each layer's reconstruction
error at its optimum,
the errors copied to the host and the K = 15 L-Layers selected there. Inputs are seeded synthetic
tensors already resident in HBM when the timed region starts. `--workload-cfg 4` runs the same step
at the 14B shape (40 layers x 40 heads, d = 5120, K = 20).

Prints one JSON line. `value` is the dual-stream attention's rate inside the step (algorithmic
4 n_q n_keys H d_h FLOP per call over the average launch time from HIP events), the metric's first
half; the absorb time per layer (statistics + solve + error), the step's own rate, the attention on
the 60-frame history (workload 5) and on the 14B shape's last warmup chunk, and the statistics
kernel's roofline are reported beside it, with the oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 (e4m3) MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (tuning only)")
    ap.add_argument("--workload-cfg", type=int, default=3, choices=(3, 4),
                    help="workload of the timed step: 3 = the Wan-1.3B warmup (default), 4 = the 14B warmup "
                         "(40 layers x 40 heads, d = 5120)")
    ap.add_argument("--stats-per-chunk", action="store_true",
                    help="update the statistics after every chunk (one batched call per chunk over that chunk's "
                         "rows, outputs reused) instead of once over the rows of all warmup chunks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the attention timings on workloads 5 and 4 that follow the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (HBM counter calibration)")
    ap.add_argument("--attn-only-cfg", type=int, default=None,
                    help="time only ispa_attn_dual on workload 2, 4 (chunk 4) or 5 (dual, local-only and "
                         "single-pass forms, warm and cold cache) and print one JSON line")
    ap.add_argument("--steady", action="store_true",
                    help="time the steady state after the warmup: L-Layer vs F-Layer chunk at 9/30/60 frames")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8-score attention against the bf16 kernel on workloads 2 and 5")
    ap.add_argument("--future", action="store_true",
                    help="time the future-query importance scores over workload 5's cache")
    ap.add_argument("--tempcache", action="store_true",
                    help="time the TempCache merge and attention over merged vs original history")
    ap.add_argument("--gram-only-cfg", type=int, default=None,
                    help="time only the statistics update of one chunk at workload 3's or 4's width")
    ap.add_argument("--gram-rows", type=int, default=None,
                    help="rows per statistics call for --gram-only-cfg (default: one chunk, 4680; the warmup "
                         "step's call takes all 4 chunks' rows, 18720)")
    ap.add_argument("--absorb-cfg", type=int, default=None,
                    help="time the whole Layer Absorb of workload 3 or 4 (all layers: statistics of the "
                         "warmup chunks, one batched solve, one batched error, ranking) per layer")
    return ap.parse_args()


def bf16_dev(x, torch):
    import ispa_inputs as inputs
    bits = inputs.bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda", non_blocking=False)


def attn_flops(n_q, n_keys, H, dh):
    return 4.0 * n_q * n_keys * H * dh


def attn_bytes(n_q, n_keys, H, dh, elem=2):
    # Q, K, V read once; A_loc, A_full written once; three LSE rows
    return elem * (n_q * H * dh + 2 * n_keys * H * dh + 2 * n_q * H * dh) + 3 * 4 * H * n_q


class Layer:
    """Device-resident inputs of one layer: the key/value cache of all 12 warmup frames and the four
    chunks' queries."""

    def __init__(self, wl, layer, torch):
        import ispa_inputs as inputs
        cache = inputs.LayerCache(wl, layer)
        self.k = bf16_dev(cache.k, torch)
        self.v = bf16_dev(cache.v, torch)
        self.q = []
        for c in range(len(wl.chunks)):
            inp = inputs.attention_inputs(wl.cfg, layer, c, cache=cache)
            self.q.append(bf16_dev(inp["q"], torch))
        self.w = torch.from_numpy(inputs.weight(wl.cfg, layer)).to("cuda")

    def seg(self, r):
        import ispa_inputs as inputs
        a, b = r[0] * inputs.FRAME_TOKENS, r[1] * inputs.FRAME_TOKENS
        return self.k[a:b], self.v[a:b]


# HBM bytes per attention launch of the warmup step (average over its 4 chunk shapes), from
# rocprofv3 FETCH_SIZE x 1.9997 + WRITE_SIZE x 1.000 (factors from a 256 MiB device copy), taken on the
# build whose attention source and build script (with its compiler flags) hash to this SHA-256
# (profiles/attn_dual_bf16_pp_wan1.3b-warmup.md). Reported only while both are unchanged.
ATTN_TRAFFIC = {"sha256": "71294b539a289b56b3f04cfd50f79d77fcb354c4871113d55b4933307ef06ee3",
                "bytes_per_launch": 157836418}


def attn_traffic():
    # keyed by the attention source and the build script (which holds its compiler flags)
    import hashlib
    h = hashlib.sha256()
    try:
        for part in (("csrc", "attn.hip"), ("build.py",)):
            with open(os.path.join(ROOT, "kv_cache_attention_split_amd", *part), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    digest = h.hexdigest()
    return ATTN_TRAFFIC["bytes_per_launch"] if digest == ATTN_TRAFFIC["sha256"] else None


# HBM bytes per statistics call of the warmup step (one batched call of the 30 layers: the 256 x 256
# tile kernel with 8 waves and its last partial round as 128 x 128 quarters), keyed by the rows per call
# (18,720: the rows of all 4 warmup chunks), from the same FETCH_SIZE / WRITE_SIZE runs and factors (both
# kernels summed), taken on the statistics source with this SHA-256; reported only while the source is
# unchanged and for a call of those rows.
GRAM_TRAFFIC = {"sha256": "92f1230a9384da7f2650c35455050235c5e5385a8b44801c213cb5c712bda26d",
                "bytes_per_launch": {18720: 20602037030}}


def gram_traffic(rows):
    import hashlib
    src = os.path.join(ROOT, "kv_cache_attention_split_amd", "csrc", "gram.hip")
    try:
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    return GRAM_TRAFFIC["bytes_per_launch"].get(rows) if digest == GRAM_TRAFFIC["sha256"] else None


def cpu_baseline(wl):
    """The oracle (fp64 NumPy) on a bounded sample of the same workload, timed on the host cores."""
    import ispa_inputs as inputs
    from oracle import absorb as oab
    from oracle import attention as oatt
    cores = len(os.sched_getaffinity(0))
    H, dh, d = wl.n_heads, wl.head_dim, wl.d
    # (a) attention of all 4680 query rows of chunk 4 (all heads, 18720 keys); at 40 heads the first
    # frame's 1560 rows, so that the sample stays within about half a minute
    inp = inputs.attention_inputs(wl.cfg, 0, 3)
    rows = np.arange(inp["q"].shape[0] if H <= 16 else inputs.FRAME_TOKENS)
    t0 = time.perf_counter()
    oatt.dual_stream(inp, rows=rows)
    t_att = time.perf_counter() - t0
    n_keys = sum(inp[k].shape[0] for k in ("sink_k", "cur_k", "hist_k"))
    f_att = attn_flops(len(rows), n_keys, H, dh)
    # (b) Layer Absorb of 8 layers: statistics over the 4 warmup chunks, solve, error
    n_abs_layers = 8 if d <= 2048 else 1
    t_abs = 0.0
    f_abs = 0.0
    for layer in range(n_abs_layers):
        chunks = [inputs.absorb_rows(wl.cfg, layer, c) for c in range(len(wl.chunks))]
        w = inputs.weight(wl.cfg, layer).astype(np.float64)
        t0 = time.perf_counter()
        st = oab.accumulate([(c["a_loc"], c["a_full"]) for c in chunks])
        dw = oab.ridge_delta_w(st["G"], st["C"], w, wl.lam)
        oab.layer_error_stats(st["G"], st["C"], st["H"], w, dw)
        t_abs += time.perf_counter() - t0
        n_rows = sum(c["a_loc"].shape[0] for c in chunks)
        f_abs += 4.0 * n_rows * d * d + 13.0 / 3.0 * d ** 3 + 4.0 * d ** 3
    return {
        "value": round((f_att + f_abs) / (t_att + t_abs) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle: dual-stream attention of {len(rows)} query rows x {H} heads "
                   f"over {n_keys} keys (chunk 4, layer 0) in {t_att:.2f} s, plus Layer Absorb of "
                   f"{n_abs_layers} layers (statistics of 4 x 4680 rows, solve, error at d={d}) in "
                   f"{t_abs:.2f} s; rate = the GPU's algorithmic FLOP count for that work / time"),
        "attn_tflops": round(f_att / t_att / 1e12, 6),
        "absorb_ms_per_layer": round(t_abs * 1e3 / n_abs_layers, 1),
        "cpu_model": _cpu_model(),
        "blas": _blas_name(),
        "brute_force": _brute_force_leg(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_name():
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:   # noqa: BLE001 - the build description is optional
        return None


def _brute_force_leg():
    """The pure-Python loop form of the oracle (one core) on 16 query rows of workload 1 (2 heads x 64,
    all 704 keys), timed on its own."""
    import ispa_inputs as inputs
    from oracle import brute
    inp = inputs.attention_inputs(1, 0, 0)
    rows = 16
    q = inp["q"][:rows].tolist()
    k = np.concatenate([inp["sink_k"], inp["cur_k"], inp["hist_k"]]).tolist()
    v = np.concatenate([inp["sink_v"], inp["cur_v"], inp["hist_v"]]).tolist()
    t0 = time.perf_counter()
    brute.attention_loops(q, k, v, float(inp["scale"]))
    t = time.perf_counter() - t0
    H, dh = inp["q"].shape[1], inp["q"].shape[2]
    return {"rows": rows, "keys": len(k), "heads": H, "head_dim": dh, "seconds": round(t, 3),
            "gflops": round(attn_flops(rows, len(k), H, dh) / t / 1e9, 4), "cores": 1}


def _time_calls(call, n, warmup, torch, cold_scratch=None):
    """Median per-call time in ms from HIP events on the current stream. With `cold_scratch`, a
    512 MiB write runs before every call so that the inputs are no longer in the caches."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for i in range(n):
        if cold_scratch is not None:
            cold_scratch.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def attn_report(cfg, steps, warmup, torch):
    """Attention on one workload in three forms, warm and cold cache:
    dual   = the dual-stream call (A_loc, A_full, three LSE rows);
    balanced = the same call with the balanced schedule over the compute units (where it applies);
    local  = local-only call (sink + current keys, A_loc and lse_loc only);
    single = one local-only call over all keys (sink and history joined into one segment), i.e.
             single-pass full attention with no merge and one output; dual / single - 1 is the
             overhead of the dual stream."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    wl = inputs.CONFIGS[cfg]
    chunk = 3 if cfg in (3, 4) else 0
    inp = inputs.attention_inputs(cfg, 0, chunk)
    dev = {k: bf16_dev(inp[k], torch) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    joined_k = torch.cat([dev["sink_k"], dev["hist_k"]], dim=0)
    joined_v = torch.cat([dev["sink_v"], dev["hist_v"]], dim=0)
    empty = dev["hist_k"][:0]
    n_q = inp["q"].shape[0]
    H, dh = wl.n_heads, wl.head_dim
    a_loc = torch.empty((n_q, H * dh), dtype=torch.bfloat16, device="cuda")
    a_full = torch.empty_like(a_loc)
    lse = [torch.empty((H, n_q), dtype=torch.float32, device="cuda") for _ in range(3)]
    n_sc = inp["sink_k"].shape[0] + inp["cur_k"].shape[0]
    n_all = n_sc + inp["hist_k"].shape[0]
    scratch = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
    calls = {
        "dual": (n_all, lambda: ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"],
                                                    dev["hist_k"], dev["hist_v"], wl.scale, a_loc, a_full,
                                                    lse[0], lse[1], lse[2])),
        "local": (n_sc, lambda: ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"],
                                                    empty, empty, wl.scale, a_loc, None, lse[0])),
        "single": (n_all, lambda: ispa.ispa_attn_dual(dev["q"], joined_k, joined_v, dev["cur_k"], dev["cur_v"],
                                                      empty, empty, wl.scale, a_loc, None, lse[0])),
    }
    ws_bytes = ispa.ispa_attn_dual_balanced_workspace(dev["q"], n_sc, n_all - n_sc)
    if ws_bytes > 0:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        calls["balanced"] = (n_all, lambda: ispa.ispa_attn_dual_balanced(
            dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"], dev["hist_k"], dev["hist_v"], wl.scale,
            a_loc, a_full, lse[0], lse[1], lse[2], ws=ws))
    # clocks ramp up over the first tenths of a second of load: run every form for about half a
    # second before timing, then time the forms in interleaved rounds and keep the median round
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:
        for _, call in calls.values():
            call()
        torch.cuda.synchronize()
    rounds = {mode: ([], []) for mode in calls}
    for _ in range(3):
        for mode, (nk, call) in calls.items():
            rounds[mode][0].append(_time_calls(call, steps, warmup, torch))
            rounds[mode][1].append(_time_calls(call, steps, warmup, torch, cold_scratch=scratch))
    res = {}
    for mode, (nk, call) in calls.items():
        fl = attn_flops(n_q, nk, H, dh)
        warm = float(np.median(rounds[mode][0]))
        cold = float(np.median(rounds[mode][1]))
        res[mode] = {"keys": nk, "warm_ms": round(warm, 4), "cold_ms": round(cold, 4),
                     "tflops_warm": round(fl / warm / 1e9, 1), "frac_warm": round(fl / warm / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "tflops_cold": round(fl / cold / 1e9, 1)}
    out = {"workload": wl.name, "n_q": n_q, "heads": H, "head_dim": dh, "attention": res,
           "dual_overhead_vs_single_pass": round(res["dual"]["warm_ms"] / res["single"]["warm_ms"] - 1.0, 4),
           "full_over_local_time": round(res["dual"]["warm_ms"] / res["local"]["warm_ms"], 3)}
    print(json.dumps(out), flush=True)


def gram_report(cfg, steps, warmup, torch, rows=None):
    """Statistics update of N rows (one 4680-row chunk unless given) at a workload's width d: one layer
    per call, and all the workload's layers in one batched call (warm median time and rate; 4 N d^2 FLOP
    per layer: G and F as half products, X in full)."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    wl = inputs.CONFIGS[cfg]
    d, n, L = wl.d, rows or inputs.CHUNK_TOKENS, wl.n_layers
    g = torch.Generator(device="cuda").manual_seed(1234 + cfg)
    a_loc = [(0.02 * torch.randn((n, d), device="cuda", generator=g)).to(torch.bfloat16) for _ in range(L)]
    a_full = [(0.02 * torch.randn((n, d), device="cuda", generator=g)).to(torch.bfloat16) for _ in range(L)]
    st = [[torch.zeros((d, d), dtype=torch.float32, device="cuda") for _ in range(3)] for _ in range(L)]
    calls = {
        "one_layer": (1, lambda: ispa.ispa_absorb_accumulate(a_loc[0], a_full[0], st[0][0], st[0][1], st[0][2])),
        "all_layers": (L, lambda: ispa.ispa_absorb_accumulate_batched(a_loc, a_full, [s[0] for s in st],
                                                                      [s[1] for s in st], [s[2] for s in st])),
    }
    out = {"workload": wl.name, "rows": n, "d": d}
    for name, (layers, call) in calls.items():
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            call()
            torch.cuda.synchronize()
        ms = float(np.median([_time_calls(call, steps, warmup, torch) for _ in range(3)]))
        fl = 4.0 * n * d * d * layers
        out[name] = {"layers": layers, "ms": round(ms, 4), "ms_per_layer": round(ms / layers, 4),
                     "tflops": round(fl / ms / 1e9, 1), "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps({"statistics": out}), flush=True)


def absorb_report(cfg, steps, warmup, torch):
    """Layer Absorb of a whole model: the statistics of its warmup chunks for every layer, one batched
    ridge solve, one batched error and the ranking (the step of workload 3 without its attention, and
    the same at the 14B shape of workload 4). Rows are drawn on the device (bf16 N(0, 0.02^2); chunks
    without history have A_full = A_loc, the others a perturbed copy), W ~ N(0, 1/d) per layer. Reports
    ms per layer for each part, its rate (statistics 4 N d^2 per chunk on bf16 matrix cores; solve
    13/3 d^3 and error 4 d^3 on fp32 matrix cores) and the selected layers."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    wl = inputs.CONFIGS[cfg]
    d, n, L = wl.d, inputs.CHUNK_TOKENS, wl.n_layers
    g = torch.Generator(device="cuda").manual_seed(4321 + cfg)
    rows = []
    for ch in wl.chunks:
        a_loc = (0.02 * torch.randn((n, d), device="cuda", generator=g)).to(torch.bfloat16)
        if ch.hist[1] > ch.hist[0]:
            a_full = (a_loc.float() + 0.005 * torch.randn((n, d), device="cuda", generator=g)).to(torch.bfloat16)
        else:
            a_full = a_loc
        rows.append((a_loc, a_full))
    Ws = [torch.randn((d, d), device="cuda", generator=g) / float(np.sqrt(d)) for _ in range(L)]
    stats = [[torch.zeros((d, d), dtype=torch.float32, device="cuda") for _ in range(3)] for _ in range(L)]
    Gs, Xs, Fs = [s_[0] for s_ in stats], [s_[1] for s_ in stats], [s_[2] for s_ in stats]
    dW = [torch.empty((d, d), dtype=torch.float32, device="cuda") for _ in range(L)]
    info = torch.zeros((L,), dtype=torch.int32, device="cuda")
    eps = torch.zeros((L,), dtype=torch.float64, device="cuda")
    ref = torch.zeros_like(eps)
    ws_solve = torch.empty(ispa.ispa_absorb_solve_workspace(d, L), dtype=torch.uint8, device="cuda")
    ws_err = torch.empty(ispa.ispa_layer_error_workspace(d, L), dtype=torch.uint8, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def run():
        for s_ in stats:
            for t in s_:
                t.zero_()
        e = [ev() for _ in range(4)]
        e[0].record()
        for li in range(L):
            for a_loc, a_full in rows:
                ispa.ispa_absorb_accumulate(a_loc, a_full, Gs[li], Xs[li], Fs[li])
        e[1].record()
        ispa.ispa_absorb_solve(Gs, Xs, Ws, dW, wl.lam, info, ws_solve)
        e[2].record()
        ispa.ispa_layer_error(Gs, Xs, Fs, Ws, dW, eps, ref, ws_err)
        e[3].record()
        sel = ispa.ispa_rank_layers(eps.cpu().numpy().tolist(), wl.k_select)
        return [e[i].elapsed_time(e[i + 1]) for i in range(3)], sel

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:
        run()
    for _ in range(warmup):
        run()
    res = [run() for _ in range(steps)]
    ms = np.median(np.array([r[0] for r in res]), axis=0) / L
    fl = (4.0 * n * d * d * len(rows), 13.0 / 3.0 * d ** 3, 4.0 * d ** 3)
    peaks = (PEAK_BF16_TFLOPS, PEAK_F32_TFLOPS, PEAK_F32_TFLOPS)
    out = {}
    for name, t, f, p in zip(("statistics", "solve", "error"), ms, fl, peaks):
        out[name] = {"ms_per_layer": round(float(t), 4), "tflops": round(f / t / 1e9, 1),
                     "frac": round(f / t / 1e9 / p, 4)}
    print(json.dumps({"workload": wl.name, "layers": L, "d": d, "chunks": len(rows), "rows_per_chunk": n,
                      "absorb_ms_per_layer": round(float(ms.sum()), 4), **out,
                      "info_nonzero": int((info != 0).sum().item()),
                      "selected_l_layers": list(res[-1][1][0])}), flush=True)


def tempcache_report(steps, warmup, torch):
    """TempCache exact merge (FAST-AR page, section 2 part A, Lemma 5.1) on workload 5's cache shape:
    12 heads x 128, 4680 queries, sink and current chunk of 4680 keys, a 60-frame history of 1560
    tokens per frame in which a fraction of token positions is static (the same key in every frame).
    Reports the merge kernel (time, HBM rate) and attention over the original history against
    attention over the merged history with its log-count bias; `bias_overhead` is the biased kernel
    over the original keys (zero bias) against the plain kernel. Inputs are drawn on the device."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    wl = inputs.CONFIGS[5]
    H, dh = wl.n_heads, wl.head_dim
    n_q = n_sink = n_cur = inputs.CHUNK_TOKENS
    frames, ft = 60, inputs.FRAME_TOKENS
    n_hist = frames * ft
    g = torch.Generator(device="cuda").manual_seed(77)

    def randn(*shape):
        return torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)

    q, sink_k, sink_v, cur_k, cur_v = (randn(n, H, dh) for n in (n_q, n_sink, n_sink, n_cur, n_cur))
    hist_v = randn(n_hist, H, dh)
    a_loc = torch.empty((n_q, H * dh), dtype=torch.bfloat16, device="cuda")
    a_full = torch.empty_like(a_loc)
    lse = [torch.empty((H, n_q), dtype=torch.float32, device="cuda") for _ in range(3)]
    zero_bias = torch.zeros(n_hist, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(5)
    reports = []
    for frac in (0.25, 0.5, 0.75):
        n_static = int(round(frac * ft))
        static_pos = np.sort(rng.choice(ft, size=n_static, replace=False))
        is_static = np.zeros(ft, dtype=bool)
        is_static[static_pos] = True
        rank = np.cumsum(is_static) - 1
        tok = np.arange(n_hist)
        pos = tok % ft
        labels = np.where(is_static[pos], rank[pos], 0)
        dyn = ~is_static[pos]
        labels[dyn] = n_static + np.arange(int(dyn.sum()))
        off, mem = inputs.csr_from_labels(labels)
        G = off.size - 1
        hist_k = randn(n_hist, H, dh)
        static_keys = randn(n_static, H, dh)
        sel = torch.from_numpy(np.nonzero(~dyn)[0]).cuda()
        hist_k[sel] = static_keys[torch.from_numpy(labels[~dyn]).cuda()]
        off_d, mem_d = torch.from_numpy(off).cuda(), torch.from_numpy(mem).cuda()
        mk = torch.empty((G, H, dh), dtype=torch.bfloat16, device="cuda")
        mv = torch.empty_like(mk)
        mb = torch.empty(G, dtype=torch.float32, device="cuda")
        calls = {
            "merge": lambda: ispa.ispa_kv_merge(hist_k, hist_v, off_d, mem_d, mk, mv, mb),
            "original": lambda: ispa.ispa_attn_dual(q, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v, wl.scale,
                                                    a_loc, a_full, lse[0], lse[1], lse[2]),
            "merged": lambda: ispa.ispa_attn_dual_biased(q, sink_k, sink_v, cur_k, cur_v, mk, mv, wl.scale,
                                                         a_loc, a_full, lse[0], lse[1], lse[2], hist_bias=mb),
            "biased_same_keys": lambda: ispa.ispa_attn_dual_biased(q, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v,
                                                                   wl.scale, a_loc, a_full, lse[0], lse[1], lse[2],
                                                                   hist_bias=zero_bias),
        }
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            for call in calls.values():
                call()
            torch.cuda.synchronize()
        ms = {k: [] for k in calls}
        for _ in range(3):
            for k, call in calls.items():
                ms[k].append(_time_calls(call, steps, warmup, torch))
        ms = {k: float(np.median(v)) for k, v in ms.items()}
        row = H * dh * 2
        merge_bytes = 2 * n_hist * row + 2 * G * row + 4 * (G + 1) + 4 * n_hist + 4 * G
        keys_orig = n_sink + n_cur + n_hist
        keys_merged = n_sink + n_cur + G
        reports.append({
            "static_frac": frac, "hist_keys": n_hist, "merged_hist_keys": G,
            "merge": {"ms": round(ms["merge"], 4), "bytes": merge_bytes,
                      "gbps": round(merge_bytes / ms["merge"] / 1e6, 1),
                      "frac_hbm": round(merge_bytes / ms["merge"] / 1e6 / PEAK_HBM_GBS, 4)},
            "attn_original_ms": round(ms["original"], 4), "attn_merged_ms": round(ms["merged"], 4),
            "attn_speedup": round(ms["original"] / ms["merged"], 3),
            "key_ratio": round(keys_orig / keys_merged, 3),
            "merged_tflops": round(attn_flops(n_q, keys_merged, H, dh) / ms["merged"] / 1e9, 1),
            "bias_overhead": round(ms["biased_same_keys"] / ms["original"] - 1.0, 4)})
        del hist_k, static_keys, mk, mv, mb
    print(json.dumps({"workload": "wan1.3b-long tempcache", "frames": frames, "frame_tokens": ft,
                      "heads": H, "head_dim": dh, "queries": n_q, "tempcache": reports}), flush=True)


def future_report(steps, warmup, torch):
    """Future-query importance of every cached key (Future Forcing page, module 1) on workload 5's
    cache: 12 heads x 128, 4680 sink + 4680 current + 93,600 history keys, proxies of one future
    chunk (4680 queries, 3 frames) or one frame (1560). Two passes (proxy log-sum-exp, then per-key
    sums); each does the 2 n_p n_k d_h FLOP of Q~ K^T per head and n_p n_k exponentials."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    wl = inputs.CONFIGS[5]
    H, dh = wl.n_heads, wl.head_dim
    n_sink = n_cur = inputs.CHUNK_TOKENS
    n_hist = 60 * inputs.FRAME_TOKENS
    n_keys = n_sink + n_cur + n_hist
    g = torch.Generator(device="cuda").manual_seed(91)

    def randn(*shape):
        return torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)

    sink_k, cur_k, hist_k = randn(n_sink, H, dh), randn(n_cur, H, dh), randn(n_hist, H, dh)
    scores = torch.empty((H, n_keys), dtype=torch.float32, device="cuda")
    token = torch.empty(n_keys, dtype=torch.float32, device="cuda")
    out = []
    for n_p in (inputs.CHUNK_TOKENS, inputs.FRAME_TOKENS):
        q = randn(n_p, H, dh)
        ws = torch.empty(ispa.ispa_future_scores_workspace(H, n_p), dtype=torch.uint8, device="cuda")
        call = lambda: ispa.ispa_future_scores(q, sink_k, cur_k, hist_k, wl.scale, scores, ws, lam=0.5,   # noqa: E731
                                               token_score=token)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            call()
            torch.cuda.synchronize()
        ms = float(np.median([_time_calls(call, steps, warmup, torch) for _ in range(3)]))
        fl = 2 * 2.0 * n_p * n_keys * dh * H          # Q~ K^T in both passes
        out.append({"proxies": n_p, "keys": n_keys, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                    "frac_mfma": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                    "gexp_per_s": round(2.0 * n_p * n_keys * H / ms / 1e6, 1)})
    print(json.dumps({"workload": "wan1.3b-long future scores", "heads": H, "head_dim": dh, "future": out}),
          flush=True)


def fp8_report(steps, warmup, torch):
    """FP8 attention scores (e4m3 q and keys, per-head scales; bf16 values) and FP8 attention with the value
    product in FP8 too (e4m3 values, per-head scales) against the bf16 kernel on workloads 2 and 5 (dual
    stream), the quantiser's rate on the keys, and the FP8 statistics of one
    4680-row chunk against the bf16 ones at workload 3's and 4's width. Attention FLOP are counted as
    for bf16 (4 n_q n_k d_h per head); statistics FLOP 4 N d^2."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    rows = []
    for cfg in (2, 5):
        wl = inputs.CONFIGS[cfg]
        inp = inputs.attention_inputs(cfg, 0, 0)
        dev = {k: bf16_dev(inp[k], torch) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
        H, dh = wl.n_heads, wl.head_dim
        n_q = inp["q"].shape[0]
        keys = torch.cat([dev["sink_k"], dev["cur_k"], dev["hist_k"]], dim=0)
        vals = torch.cat([dev["sink_v"], dev["cur_v"], dev["hist_v"]], dim=0)
        q_s = torch.empty(H, dtype=torch.float32, device="cuda")
        k_s = torch.empty(H, dtype=torch.float32, device="cuda")
        v_s = torch.empty(H, dtype=torch.float32, device="cuda")
        ispa.ispa_fp8_head_scales(dev["q"], q_s)
        ispa.ispa_fp8_head_scales(keys, k_s)
        ispa.ispa_fp8_head_scales(vals, v_s)
        q8 = torch.empty(dev["q"].shape, dtype=torch.uint8, device="cuda")
        ispa.ispa_fp8_quantize(dev["q"], q_s, q8)
        k8, v8 = {}, {}
        for n in ("sink", "cur", "hist"):
            k8[n] = torch.empty(dev[n + "_k"].shape, dtype=torch.uint8, device="cuda")
            ispa.ispa_fp8_quantize(dev[n + "_k"], k_s, k8[n])
            v8[n] = torch.empty(dev[n + "_v"].shape, dtype=torch.uint8, device="cuda")
            ispa.ispa_fp8_quantize(dev[n + "_v"], v_s, v8[n])
        a_loc = torch.empty((n_q, H * dh), dtype=torch.bfloat16, device="cuda")
        a_full = torch.empty_like(a_loc)
        lse = [torch.empty((H, n_q), dtype=torch.float32, device="cuda") for _ in range(3)]
        calls = {
            "bf16": lambda: ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"],
                                                dev["hist_k"], dev["hist_v"], wl.scale, a_loc, a_full, *lse),
            "fp8": lambda: ispa.ispa_attn_dual_fp8(q8, q_s, k8["sink"], dev["sink_v"], k8["cur"], dev["cur_v"],
                                                   k8["hist"], dev["hist_v"], k_s, wl.scale, a_loc, a_full, *lse),
            "fp8_pv": lambda: ispa.ispa_attn_dual_fp8_pv(q8, q_s, k8["sink"], v8["sink"], k8["cur"], v8["cur"],
                                                         k8["hist"], v8["hist"], k_s, v_s, wl.scale, a_loc, a_full,
                                                         *lse),
            "quantize_keys": lambda: ispa.ispa_fp8_quantize(keys, k_s, torch.empty(keys.shape, dtype=torch.uint8,
                                                                                   device="cuda")),
        }
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            for c in calls.values():
                c()
            torch.cuda.synchronize()
        ms = {k: float(np.median([_time_calls(c, steps, warmup, torch) for _ in range(3)])) for k, c in calls.items()}
        n_keys = keys.shape[0]
        fl = attn_flops(n_q, n_keys, H, dh)
        qbytes = n_keys * H * dh * 3          # bf16 read + e4m3 write
        rows.append({"workload": wl.name, "keys": n_keys, "bf16_ms": round(ms["bf16"], 4),
                     "fp8_ms": round(ms["fp8"], 4), "speedup": round(ms["bf16"] / ms["fp8"], 3),
                     "fp8_tflops_bf16_count": round(fl / ms["fp8"] / 1e9, 1),
                     "fp8_pv_ms": round(ms["fp8_pv"], 4), "fp8_pv_speedup": round(ms["bf16"] / ms["fp8_pv"], 3),
                     "fp8_pv_tflops_bf16_count": round(fl / ms["fp8_pv"] / 1e9, 1),
                     "fp8_pv_frac_fp8_peak": round(fl / ms["fp8_pv"] / 1e9 / PEAK_FP8_TFLOPS, 4),
                     "quantize_keys_ms": round(ms["quantize_keys"], 4),
                     "quantize_gbps": round(qbytes / ms["quantize_keys"] / 1e6, 1)})
    stats = []
    for cfg in (3, 4):
        wl = inputs.CONFIGS[cfg]
        d, n, hd = wl.d, inputs.CHUNK_TOKENS, wl.head_dim
        g = torch.Generator(device="cuda").manual_seed(4321 + cfg)
        a_loc = (0.02 * torch.randn((n, d), device="cuda", generator=g)).to(torch.bfloat16)
        a_full = (0.02 * torch.randn((n, d), device="cuda", generator=g)).to(torch.bfloat16)
        H = d // hd
        s_loc = torch.empty(H, dtype=torch.float32, device="cuda")
        s_full = torch.empty_like(s_loc)
        ispa.ispa_fp8_head_scales(a_loc.view(n, H, hd), s_loc)
        ispa.ispa_fp8_head_scales(a_full.view(n, H, hd), s_full)
        c_loc = torch.empty((n, H, hd), dtype=torch.uint8, device="cuda")
        c_full = torch.empty_like(c_loc)
        ispa.ispa_fp8_quantize(a_loc.view(n, H, hd), s_loc, c_loc)
        ispa.ispa_fp8_quantize(a_full.view(n, H, hd), s_full, c_full)
        st = [torch.zeros((d, d), dtype=torch.float32, device="cuda") for _ in range(3)]
        calls = {"bf16": lambda: ispa.ispa_absorb_accumulate(a_loc, a_full, st[0], st[1], st[2]),
                 "fp8": lambda: ispa.ispa_absorb_accumulate_fp8(c_loc.view(n, d), s_loc, c_full.view(n, d), s_full,
                                                                hd, st[0], st[1], st[2])}
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            for c in calls.values():
                c()
            torch.cuda.synchronize()
        ms = {k: float(np.median([_time_calls(c, steps, warmup, torch) for _ in range(3)])) for k, c in calls.items()}
        fl = 4.0 * n * d * d
        stats.append({"workload": wl.name, "rows": n, "d": d, "bf16_ms": round(ms["bf16"], 4),
                      "fp8_ms": round(ms["fp8"], 4), "speedup": round(ms["bf16"] / ms["fp8"], 3),
                      "fp8_tflops": round(fl / ms["fp8"] / 1e9, 1)})
    print(json.dumps({"fp8_attention": rows, "fp8_statistics": stats}), flush=True)


def steady_report(steps, warmup, torch):
    """After the warmup (ISPA stage 3): time of one chunk of an L-Layer (local-only attention over sink
    + current chunk, projection with W + dW) against an F-Layer (full attention over the whole cache,
    projection with W), at 9, 30 and 60 frames of history (workload 5's tensors), and the per-chunk
    model time with K of N layers converted."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    wl5 = inputs.CONFIGS[5]
    wl3 = inputs.CONFIGS[3]
    inp = inputs.attention_inputs(5, 0, 0)
    dev = {k: bf16_dev(inp[k], torch) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
    n_q = inp["q"].shape[0]
    H, dh = wl5.n_heads, wl5.head_dim
    d = H * dh
    empty = dev["hist_k"][:0]
    a = torch.empty((n_q, d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(a)
    lse = torch.empty((H, n_q), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    w = (torch.randn((d, d), device="cuda", generator=g) / d ** 0.5).float()
    dw = (1e-2 * torch.randn((d, d), device="cuda", generator=g) / d ** 0.5).float()
    w_new = torch.empty((d, d), dtype=torch.bfloat16, device="cuda")
    w_old = torch.empty((d, d), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_apply_delta(w, dw, w_new)
    ispa.ispa_apply_delta(w, torch.zeros_like(dw), w_old)
    t_apply = _time_calls(lambda: ispa.ispa_apply_delta(w, dw, w_new), steps, warmup, torch)
    frame = inputs.FRAME_TOKENS
    n_sc = inp["sink_k"].shape[0] + inp["cur_k"].shape[0]

    def local_layer():
        ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"], dev["cur_v"], empty, empty,
                            wl5.scale, a, None, lse)
        ispa.ispa_project(a, w_new, y)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:
        local_layer()
        torch.cuda.synchronize()
    t_proj = _time_calls(lambda: ispa.ispa_project(a, w_new, y), steps, warmup, torch)
    t_l = _time_calls(local_layer, steps, warmup, torch)
    rows = []
    for frames in (9, 30, 60):
        nh = frames * frame
        jk = torch.cat([dev["sink_k"], dev["hist_k"][:nh]], dim=0)
        jv = torch.cat([dev["sink_v"], dev["hist_v"][:nh]], dim=0)

        def full_layer():
            ispa.ispa_attn_dual(dev["q"], jk, jv, dev["cur_k"], dev["cur_v"], empty, empty, wl5.scale, a, None, lse)
            ispa.ispa_project(a, w_old, y)

        t_f = _time_calls(full_layer, steps, warmup, torch)
        n_layers, k = wl3.n_layers, wl3.k_select
        rows.append({"history_frames": frames, "keys_full": n_sc + nh, "keys_local": n_sc,
                     "f_layer_ms": round(t_f, 4), "l_layer_ms": round(t_l, 4),
                     "chunk_ms_all_f": round(n_layers * t_f, 3),
                     "chunk_ms_with_l": round((n_layers - k) * t_f + k * t_l, 3),
                     "speedup": round(n_layers * t_f / ((n_layers - k) * t_f + k * t_l), 3),
                     "kv_tokens_kept_fraction": round(((n_layers - k) * (n_sc + nh) + k * n_sc)
                                                      / (n_layers * (n_sc + nh)), 4)})
        del jk, jv
    fl = 2.0 * n_q * d * d
    print(json.dumps({"workload": "wan1.3b steady state (after the warmup)", "n_q": n_q, "d": d,
                      "layers": wl3.n_layers, "l_layers": wl3.k_select,
                      "projection": {"ms": round(t_proj, 4), "tflops": round(fl / t_proj / 1e9, 1),
                                     "frac": round(fl / t_proj / 1e9 / PEAK_BF16_TFLOPS, 4)},
                      "apply_delta_ms": round(t_apply, 4), "per_history": rows}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the sharding is a design note); --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa

    if args.attn_only_cfg is not None:
        attn_report(args.attn_only_cfg, max(args.steps, 20), max(args.warmup, 5), torch)
        return
    if args.steady:
        steady_report(max(args.steps, 20), max(args.warmup, 5), torch)
        return
    if args.fp8:
        fp8_report(max(args.steps, 20), max(args.warmup, 5), torch)
        return
    if args.future:
        future_report(max(args.steps, 20), max(args.warmup, 5), torch)
        return
    if args.tempcache:
        tempcache_report(max(args.steps, 20), max(args.warmup, 5), torch)
        return
    if args.gram_only_cfg is not None:
        gram_report(args.gram_only_cfg, max(args.steps, 20), max(args.warmup, 5), torch, args.gram_rows)
        return
    if args.absorb_cfg is not None:
        absorb_report(args.absorb_cfg, min(args.steps, 5), min(args.warmup, 1), torch)
        return

    if args.calibrate_copy:
        src = torch.ones((256 << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = inputs.CONFIGS[args.workload_cfg]
    n_layers = args.layers or wl.n_layers
    H, dh, d = wl.n_heads, wl.head_dim, wl.d
    n_q = inputs.CHUNK_TOKENS

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(os.sched_getaffinity(0)))) as ex:
        layers = list(ex.map(lambda l: Layer(wl, l, torch), range(n_layers)))
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t0

    # each layer's attention outputs: the rows of all warmup chunks side by side (chunk c writes rows
    # [c n_q, (c + 1) n_q)), taken by one statistics call after the last chunk; with --stats-per-chunk
    # one chunk's rows, taken after every chunk
    n_ch = len(wl.chunks)
    per_chunk = args.stats_per_chunk
    rows_kept = n_q if per_chunk else n_ch * n_q
    a_loc = [torch.empty((rows_kept, d), dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    a_full = [torch.empty_like(x) for x in a_loc]
    row0 = [0 if per_chunk else c * n_q for c in range(n_ch)]
    lse = [torch.empty((H, n_q), dtype=torch.float32, device="cuda") for _ in range(3)]
    # every layer's G, X, F in one allocation, so that the warmup's start clears them with one fill
    stats_all = torch.zeros((n_layers, 3, d, d), dtype=torch.float32, device="cuda")
    stats = [[stats_all[li, j] for j in range(3)] for li in range(n_layers)]
    dW = [torch.empty((d, d), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    info = torch.zeros((n_layers,), dtype=torch.int32, device="cuda")
    eps = torch.zeros((n_layers,), dtype=torch.float64, device="cuda")
    ref = torch.zeros((n_layers,), dtype=torch.float64, device="cuda")
    ws_solve = torch.empty(ispa.ispa_absorb_solve_eps_workspace(d, n_layers), dtype=torch.uint8, device="cuda")
    Gs = [s[0] for s in stats]
    Xs = [s[1] for s in stats]
    Fs = [s[2] for s in stats]
    Ws = [L.w for L in layers]

    seg_keys = [sum(wl.segment_sizes(c)[k] for k in ("n_sink", "n_cur", "n_hist"))
                for c in range(len(wl.chunks))]
    flops_attn = sum(attn_flops(n_q, nk, H, dh) for nk in seg_keys) * n_layers
    flops_stats = 4.0 * n_q * d * d * n_layers * n_ch
    flops_stats_launch = flops_stats / n_ch if per_chunk else flops_stats   # one batched call
    flops_solve = 13.0 / 3.0 * d ** 3 * n_layers
    flops_err = 1.0 * d ** 3 * n_layers                     # W W^T, lower tiles
    flops_step = flops_attn + flops_stats + flops_solve + flops_err

    # the event-timed pass takes its events from a pool made beforehand: creating two timing events per
    # launch inside the pass (host work between the launches) let the queue run dry in a fresh process,
    # and the idle gaps then counted in the launches' times (attention read 40 % low)
    n_events = 2 * (n_layers * n_ch + n_ch + 1)
    pool = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    for e in pool:
        e.record()                  # the device events are made at the first record
    torch.cuda.synchronize()
    pool_it = iter(())
    ev = lambda: next(pool_it)   # noqa: E731
    timing = {"attn": [], "stats": [], "solve": []}

    def step(record: bool):
        stats_all.zero_()
        for c, ch in enumerate(wl.chunks):
            for li, L in enumerate(layers):
                sk, sv = L.seg(ch.sink)
                ck, cv = L.seg(ch.cur)
                hk, hv = L.seg(ch.hist)
                if record:
                    e0, e1 = ev(), ev()
                    e0.record()
                ispa.ispa_attn_dual(L.q[c], sk, sv, ck, cv, hk, hv, wl.scale, a_loc[li][row0[c]:row0[c] + n_q],
                                    a_full[li][row0[c]:row0[c] + n_q], lse[0], lse[1], lse[2])
                if record:
                    e1.record()
                    timing["attn"].append((e0, e1, seg_keys[c]))
            if per_chunk or c == n_ch - 1:
                if record:
                    e0, e1 = ev(), ev()
                    e0.record()
                ispa.ispa_absorb_accumulate_batched(a_loc, a_full, Gs, Xs, Fs)
                if record:
                    e1.record()
                    timing["stats"].append((e0, e1))
        if record:
            e3, e4 = ev(), ev()
            e3.record()
        ispa.ispa_absorb_solve_eps(Gs, Xs, Fs, Ws, dW, wl.lam, info, eps, ref, ws_solve)
        if record:
            e4.record()
            timing["solve"].append((e3, e4))
        eps_host = eps.cpu().numpy()        # synchronises: the ranking runs on the host
        return ispa.ispa_rank_layers(eps_host.tolist(), min(wl.k_select, n_layers))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        sel, flags = step(False)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-kernel event timing: a separate pass (so the step timing above carries no event overhead),
    # taken after the timed steps
    pool_it = iter(pool)
    step(True)
    torch.cuda.synchronize()
    att = [(a.elapsed_time(b), nk) for a, b, nk in timing["attn"]]
    att_ms = sum(t for t, _ in att)
    att_avg_ms = att_ms / len(att)
    att_flops_per_launch = flops_attn / len(att)
    stats_ms = sum(a.elapsed_time(b) for a, b in timing["stats"])
    stats_avg_ms = stats_ms / len(timing["stats"])
    solve_ms = sum(a.elapsed_time(b) for a, b in timing["solve"])

    att_tflops = att_flops_per_launch / att_avg_ms / 1e9
    stats_tflops = flops_stats_launch / stats_avg_ms / 1e9
    info_h = info.cpu().tolist()
    eps_h = eps.cpu().tolist()
    ref_h = ref.cpu().tolist()
    del a_loc, a_full, stats, Gs, Xs, Fs, dW, ws_solve
    torch.cuda.empty_cache()
    extra = {} if args.no_extra else extra_attention(wl.cfg, torch)
    out = {
        "metric": "dual-stream attn TFLOP/s (% MFMA peak); ΔW absorb ms/layer, 1.3B shape",
        "value": round(att_tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) queries/values, AR(1) rho=0.95 keys across latent frames, W ~ N(0,1/d))",
        "config": {"workload": wl.name, "layers": n_layers, "chunks": len(wl.chunks),
                   "heads": H, "head_dim": dh, "queries_per_chunk": n_q,
                   "keys_per_chunk": seg_keys, "lambda": wl.lam, "k_select": min(wl.k_select, n_layers),
                   "statistics": "per chunk" if per_chunk else "once over all warmup rows"},
        "attn_tflops": round(att_tflops, 1),
        "attn_frac_mfma_peak": round(att_tflops / PEAK_BF16_TFLOPS, 4),
        "attn_ms_per_layer": round(att_ms / n_layers, 4),
        "absorb_ms_per_layer": round((stats_ms + solve_ms) / n_layers, 4),
        "absorb_breakdown_ms_per_layer": {"statistics": round(stats_ms / n_layers, 4),
                                          "solve_and_error": round(solve_ms / n_layers, 4)},
        "stats_tflops": round(stats_tflops, 1),
        "step_tflops": round(flops_step / ms_step / 1e9, 2),
        "solve_info_nonzero": int(sum(1 for x in info_h if x != 0)),
        "eps_over_ref": [round(e / r, 6) for e, r in zip(eps_h, ref_h)][:4],
        "selected_l_layers": sel,
        "roofline": {"kernel": "attn_dual_bf16_pp_kernel", "bound": "mfma",
                     "achieved": round(att_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": attn_traffic() if wl.cfg == 3 else None,
                     "avg_launch_ms": round(att_avg_ms, 5),
                     "flops_per_launch": att_flops_per_launch},
        "roofline_statistics": {"kernel": stats_kernel_name(d, n_layers), "bound": "mfma",
                                "achieved": round(stats_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(stats_tflops / PEAK_BF16_TFLOPS, 4),
                                "traffic": gram_traffic(rows_kept) if wl.cfg == 3 and n_layers == wl.n_layers else None,
                                "avg_launch_ms": round(stats_avg_ms, 5),
                                "rows_per_launch": rows_kept,
                                "flops_per_launch": flops_stats_launch},
        **extra,
        "setup_s": round(t_setup, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


def stats_kernel_name(d, n_layers):
    """The statistics kernels one batched call of n_layers layers at width d runs (the library's rule:
    256 x 256 tiles once a launch of up to 48 layers has 512 of them, their last partial round of 256
    workgroups as quarters on the 128 x 128 kernel)."""
    T = (d + 255) // 256
    n_wide = (T * (T + 1) + T * T) * min(n_layers, 48)
    if n_wide < 512:
        return "gram_bf16_kernel"
    return "gram_bf16_wide_kernel" + (" + gram_bf16_kernel (last partial round)" if n_wide % 256 else "")


def extra_attention(step_cfg, torch):
    """Dual-stream attention on the other workloads the metric names, timed after the step (HIP events,
    median of 20 calls after a half-second warm-up each): the 60-frame history (workload 5, dual and
    local-only) and the 14B shape's last warmup chunk (workload 4 chunk 4, layer 0); on both, also the
    FP8 form with e4m3 q, keys and values (per-head scales computed and codes written on the device
    before timing; FLOP counted as for bf16, fraction of the FP8 peak)."""
    import ispa_inputs as inputs
    import kv_cache_attention_split_amd as ispa
    out = {}
    cases = [(5, 0, "attn_wan1.3b_long"), (4, 3, "attn_wan14b_chunk4")]
    for cfg, chunk, key in cases:
        wl = inputs.CONFIGS[cfg]
        inp = inputs.attention_inputs(cfg, 0, chunk)
        dev = {k: bf16_dev(inp[k], torch) for k in ("q", "sink_k", "sink_v", "cur_k", "cur_v", "hist_k", "hist_v")}
        n_q = inp["q"].shape[0]
        H, dh = wl.n_heads, wl.head_dim
        a_l = torch.empty((n_q, H * dh), dtype=torch.bfloat16, device="cuda")
        a_f = torch.empty_like(a_l)
        lse = [torch.empty((H, n_q), dtype=torch.float32, device="cuda") for _ in range(3)]
        empty = dev["hist_k"][:0]
        n_sc = inp["sink_k"].shape[0] + inp["cur_k"].shape[0]
        n_all = n_sc + inp["hist_k"].shape[0]
        forms = {"dual": (n_all, lambda: ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"],
                                                             dev["cur_v"], dev["hist_k"], dev["hist_v"], wl.scale,
                                                             a_l, a_f, lse[0], lse[1], lse[2]))}
        if cfg == 5:
            forms["local"] = (n_sc, lambda: ispa.ispa_attn_dual(dev["q"], dev["sink_k"], dev["sink_v"], dev["cur_k"],
                                                                dev["cur_v"], empty, empty, wl.scale, a_l, None, lse[0]))

        def e4m3(x):
            sc = torch.empty(H, dtype=torch.float32, device="cuda")
            ispa.ispa_fp8_head_scales(x, sc)
            codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
            ispa.ispa_fp8_quantize(x, sc, codes)
            return sc, codes
        q_s, q8 = e4m3(dev["q"])
        k_s, k8 = e4m3(torch.cat([dev["sink_k"], dev["cur_k"], dev["hist_k"]]))
        v_s, v8 = e4m3(torch.cat([dev["sink_v"], dev["cur_v"], dev["hist_v"]]))
        b = [0, inp["sink_k"].shape[0], n_sc, n_all]
        seg8 = [(k8[b[i]:b[i + 1]], v8[b[i]:b[i + 1]]) for i in range(3)]
        forms["fp8_values"] = (n_all, lambda: ispa.ispa_attn_dual_fp8_pv(
            q8, q_s, seg8[0][0], seg8[0][1], seg8[1][0], seg8[1][1], seg8[2][0], seg8[2][1], k_s, v_s, wl.scale,
            a_l, a_f, lse[0], lse[1], lse[2]))
        res = {"workload": wl.name, "n_q": n_q, "heads": H}
        for form, (nk, call) in forms.items():
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.5:
                call()
                torch.cuda.synchronize()
            ms = _time_calls(call, 20, 2, torch)
            tf = attn_flops(n_q, nk, H, dh) / ms / 1e9
            res[form] = {"keys": nk, "ms": round(ms, 4), "tflops": round(tf, 1),
                         "frac_mfma_peak": round(tf / (PEAK_FP8_TFLOPS if form == "fp8_values" else PEAK_BF16_TFLOPS), 4)}
        if "local" in res:
            res["full_over_local_time"] = round(res["dual"]["ms"] / res["local"]["ms"], 3)
        res["fp8_values_speedup"] = round(res["dual"]["ms"] / res["fp8_values"]["ms"], 3)
        out[key] = res
        del dev, a_l, a_f, lse
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
