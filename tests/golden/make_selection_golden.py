"""Write the oracle's per-layer reconstruction errors and layer selections for whole-model warmups.

    python tests/golden/make_selection_golden.py [--only NAME] [--workers N]

Calls only `oracle/` and `ispa_inputs/` (never the HIP library), so every stored value is the
oracle's. Source: ISPA summary page ("Instance-Specific Parametric Absorption"), section 2 "Framework
Core": stage 1 "Dual-Stream Warmup" (A_loc, A_full of every warmup chunk), stage 2 "Layer Absorb"
(closed-form dW, first and second display equations) and "Dynamic Layer Selection" (rank layers by
reconstruction error, the K lowest become L-Layers).

Files written (tests/golden/selection_<name>.json):
  wan1.3b-warmup-attention  30 layers, 12 x 128 heads (d = 1536), the 4-chunk warmup; every layer's
                            A_loc / A_full by the oracle's attention in float64 from the seeded bf16
                            inputs (`ispa_inputs.attention_inputs`), statistics of those rows, LU
                            solve, eps on the rows; K = 15
  wan14b-warmup-rows        40 layers at d = 5120, 4 chunks of 4680 seeded rows per layer
                            (`ispa_inputs.absorb_rows`, bf16 values); K = 20
  wan14b-warmup-attention   layers 0 and 1 of the 14B warmup (40 x 128 heads), the oracle's whole
                            chain as for the 1.3B file (eps only; no selection)

Admissible selections (reading of the page's "lowest error" when two errors agree within the
tolerance): with the eps gate tol and r = (1 + tol) / (1 - tol), a set S of K layers is admissible
when max_{i in S} eps_i <= r * min_{j not in S} eps_j on the oracle's eps. Each file lists the layers
every admissible set holds (`must_select`) and those some admissible set may hold (`may_select`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import ispa_inputs as inputs  # noqa: E402
from oracle import absorb as oab  # noqa: E402
from oracle import attention as oatt  # noqa: E402

EPS_TOL = 1e-3
CITE = ("ISPA summary page (Instance-Specific Parametric Absorption), section 2 'Framework Core': stage 1 "
        "'Dual-Stream Warmup', stage 2 'Layer Absorb' (objective and closed form, first and second display "
        "equations), 'Dynamic Layer Selection' (layers ranked by reconstruction error, the lowest become L-Layers)")


def _limit_threads(n):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(n)
    except Exception:
        pass


def _absorb(cfg, layer, a_loc, a_full, with_kappa):
    wl = inputs.CONFIGS[cfg]
    st = oab.grams(a_loc, a_full)
    W = inputs.weight(cfg, layer)
    dW = oab.ridge_delta_w(st["G"], st["C"], W, wl.lam)
    out = {"layer": layer,
           "eps": oab.layer_error_rows(a_loc, a_full, W, dW),
           "ref": oab.reference_energy(st["F"], W),
           "dw_fro": float(np.linalg.norm(dW))}
    if with_kappa:
        out["kappa"] = float(np.linalg.cond(st["G"] + wl.lam * np.eye(st["G"].shape[0])))
    return out


def chain_attention(args):
    """The oracle's whole chain for one layer: attention of every warmup chunk, statistics, dW, eps."""
    cfg, layer, threads = args
    _limit_threads(threads)
    wl = inputs.CONFIGS[cfg]
    cache = inputs.LayerCache(wl, layer)
    locs, fulls = [], []
    for c in range(len(wl.chunks)):
        o = oatt.dual_stream(inputs.attention_inputs(cfg, layer, c, cache=cache))
        locs.append(o["A_loc"])
        fulls.append(o["A_full"])
    return _absorb(cfg, layer, np.concatenate(locs), np.concatenate(fulls), wl.d <= 2048)


def chain_rows(args):
    """Absorb of one layer from the seeded rows of every warmup chunk."""
    cfg, layer, threads = args
    _limit_threads(threads)
    wl = inputs.CONFIGS[cfg]
    chunks = [inputs.absorb_rows(cfg, layer, c) for c in range(len(wl.chunks))]
    a_loc = np.concatenate([c["a_loc"] for c in chunks]).astype(np.float64)
    a_full = np.concatenate([c["a_full"] for c in chunks]).astype(np.float64)
    return _absorb(cfg, layer, a_loc, a_full, wl.d <= 2048)


def admissible(eps, k, tol=EPS_TOL):
    """(oracle selection, must_select, may_select) under the tolerance rule of the module docstring."""
    eps = np.asarray(eps, dtype=np.float64)
    sel, _ = oab.rank_layers(eps, k)
    if k == 0 or k == len(eps):
        return sel.tolist(), sorted(sel.tolist()), []
    r = (1.0 + tol) / (1.0 - tol)
    srt = np.sort(eps)
    e_k, e_k1 = srt[k - 1], srt[k]
    must = [int(i) for i in range(len(eps)) if eps[i] <= e_k and e_k1 > r * eps[i]]
    may = [int(i) for i in range(len(eps)) if i not in must and eps[i] <= r * e_k]
    return [int(i) for i in sel], sorted(must), sorted(may)


SETS = {
    "wan1.3b-warmup-attention": dict(cfg=3, layers=list(range(30)), fn=chain_attention, select=True,
                                     rows="oracle attention of the 4 warmup chunks (4680 queries each; "
                                          "0/4680/9360/14040 + 4680 keys) from ispa_inputs.attention_inputs"),
    "wan14b-warmup-rows": dict(cfg=4, layers=list(range(40)), fn=chain_rows, select=True,
                               rows="ispa_inputs.absorb_rows(4, layer, chunk) for chunks 0-3 (4680 rows each, "
                                    "bf16 values, d = 5120)"),
    "wan14b-warmup-attention": dict(cfg=4, layers=[0, 1], fn=chain_attention, select=False,
                                    rows="oracle attention of the 4 warmup chunks at 40 x 128 heads from "
                                         "ispa_inputs.attention_inputs"),
}


def make(name, workers):
    spec = SETS[name]
    cfg = spec["cfg"]
    wl = inputs.CONFIGS[cfg]
    n = len(spec["layers"])
    workers = max(1, min(workers, n))
    threads = max(1, (os.cpu_count() or 1) // workers)
    t0 = time.time()
    with ProcessPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(spec["fn"], [(cfg, l, threads) for l in spec["layers"]]))
    res.sort(key=lambda r: r["layer"])
    out = {
        "what": f"oracle per-layer reconstruction error of the {wl.name} workload ({n} layers, d = {wl.d})",
        "cite": CITE,
        "generator": "tests/golden/make_selection_golden.py (oracle/ and ispa_inputs/ only)",
        "seed_base": inputs.SEED_BASE,
        "workload": wl.name,
        "cfg": cfg,
        "d": wl.d,
        "n_heads": wl.n_heads,
        "head_dim": wl.head_dim,
        "lam": wl.lam,
        "rows": spec["rows"],
        "chunks": len(wl.chunks),
        "layers": [r["layer"] for r in res],
        "eps": [r["eps"] for r in res],
        "ref": [r["ref"] for r in res],
        "dw_fro": [r["dw_fro"] for r in res],
        "eps_tol": EPS_TOL,
    }
    if "kappa" in res[0]:
        out["kappa"] = [r["kappa"] for r in res]
    if spec["select"]:
        k = wl.k_select
        sel, must, may = admissible(out["eps"], k)
        out.update({"k": k, "selected": sel, "must_select": must, "may_select": may,
                    "admissible_rule": "|S| = k and max_{i in S} eps_i <= (1 + tol) / (1 - tol) * min_{j not in S} eps_j"})
    path = os.path.join(HERE, f"selection_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"{path}: {n} layers in {time.time() - t0:.0f} s", flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", choices=sorted(SETS), action="append")
    ap.add_argument("--workers", type=int, default=max(1, (os.cpu_count() or 1)))
    a = ap.parse_args(argv)
    for name in (a.only or list(SETS)):
        make(name, a.workers)


if __name__ == "__main__":
    main()
