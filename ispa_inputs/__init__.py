"""Seeded synthetic inputs for the ISPA hot path, shared by the oracle tests and the GPU path.

This module draws random tensors and nothing else: it holds none of the method's arithmetic
(no attention, no Gram products, no solve). Both the fp64 CPU oracle and the HIP library are fed
from here, so that the two sides see identical values.

Workloads (shapes of Wan-1.3B / Wan-14B-like self-attention layers in a streaming video generator,
as used by the ISPA summary page, "Instance-Specific Parametric Absorption", section 2 "Framework
Core" and section 4 "Experimental Results"; the pages fix no tensor shapes, so the shapes below are
the workload definitions this library is measured on):

  cfg 1  fp32, 2 heads x 64 (d=128), 128 queries; 64 sink / 128 current / 512 history keys, iid N(0,1)
  cfg 2  bf16, 12 x 128 (d=1536), one 3-frame chunk (4680 queries) = warmup chunk 4:
         sink = frames 0-2, current = frames 9-11, history = frames 3-8 (9360 keys)
  cfg 3  bf16, 30 layers of cfg 2's shape, 4 warmup chunks (T_warm = 12 latent frames)
  cfg 4  bf16, 40 layers, 40 x 128 (d=5120), the 4-chunk warmup of cfg 3
  cfg 5  bf16, 12 x 128, sink = frames 0-2, current = frames 63-65, history = frames 3-62 (93600)

A latent frame holds 1560 tokens and a chunk holds 3 frames. Keys follow one AR(1) chain per
(token position, head, channel) across all latent frames in temporal order,
k_t = rho * k_{t-1} + sqrt(1 - rho^2) * z_t with rho = 0.95 and k_0 ~ N(0,1), so every key stays
N(0,1) while neighbouring frames are correlated. Queries and values are iid N(0,1). Weights W are
N(0, 1/d). bf16 workloads round every drawn value to bf16 (round to nearest even) and the rounded
values are the inputs of both sides.

TempCache merge cases (`static_history_case`) draw a history whose static token positions repeat
the same keys in every frame (the exact-duplicate case of the FAST-AR page's Lemma 5.1), with the
grouping of the history tokens in compressed form (`csr_from_labels`).

Seeds: numpy SeedSequence([base, cfg, layer, stream]) with stream 1 = key chain, 2 = values,
3 = weight, 16 + c = queries of chunk c, 32 + c = synthetic absorb rows of chunk c.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

FRAME_TOKENS = 1560
FRAMES_PER_CHUNK = 3
CHUNK_TOKENS = FRAME_TOKENS * FRAMES_PER_CHUNK  # 4680
AR_RHO = 0.95
SEED_BASE = int(os.environ.get("ISPA_SEED_BASE", "0"))

STREAM_K, STREAM_V, STREAM_W = 1, 2, 3
STREAM_Q0 = 16
STREAM_ABSORB0 = 32


# ----------------------------------------------------------------------------------------------
# bf16 rounding (input precision, not method arithmetic)
# ----------------------------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bf16-rounded values of x."""
    return bf16_bits_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------------------------
# Workload records
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Chunk:
    """Key segments of one query chunk, as latent-frame ranges [start, stop) of the layer's cache.

    `cur` is also the query range. Empty ranges mean an empty segment. `n_*_iid` override the
    frame ranges with plain token counts (cfg 1 has no frame structure).
    """
    sink: tuple
    cur: tuple
    hist: tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    dtype: str          # "f32" or "bf16"
    n_heads: int
    head_dim: int
    n_layers: int
    chunks: tuple       # tuple[Chunk]; frame ranges
    lam: float = 1e-2
    k_select: int = 0
    iid_tokens: Optional[tuple] = None   # (n_q, n_sink, n_cur, n_hist) for frame-less workloads

    @property
    def d(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def segment_sizes(self, chunk: int = 0) -> Dict[str, int]:
        if self.iid_tokens is not None:
            n_q, n_s, n_c, n_h = self.iid_tokens
            return {"n_q": n_q, "n_sink": n_s, "n_cur": n_c, "n_hist": n_h}
        ch = self.chunks[chunk]
        f = lambda r: (r[1] - r[0]) * FRAME_TOKENS
        return {"n_q": f(ch.cur), "n_sink": f(ch.sink), "n_cur": f(ch.cur), "n_hist": f(ch.hist)}

    def n_frames(self) -> int:
        return max(max(c.sink[1], c.cur[1], c.hist[1]) for c in self.chunks)


def warmup_chunks(n_chunks: int = 4) -> tuple:
    """The T_warm = 12 latent-frame warmup as 4 chunks of 3 frames.

    Chunk 0 is itself the sink (attend to it once, as the current chunk, with no separate sink).
    Chunk c >= 1: sink = frames 0-2, current = frames 3c..3c+2, history = frames 3..3c-1.
    """
    out = [Chunk(sink=(0, 0), cur=(0, 3), hist=(0, 0))]
    for c in range(1, n_chunks):
        out.append(Chunk(sink=(0, 3), cur=(3 * c, 3 * c + 3), hist=(3, 3 * c)))
    return tuple(out)


CONFIGS: Dict[int, Workload] = {
    1: Workload(1, "tiny-fp32", "f32", 2, 64, 1, (Chunk((0, 0), (0, 0), (0, 0)),),
                lam=1e-2, k_select=1, iid_tokens=(128, 64, 128, 512)),
    2: Workload(2, "wan1.3b-chunk4", "bf16", 12, 128, 1,
                (Chunk(sink=(0, 3), cur=(9, 12), hist=(3, 9)),), lam=1e-2, k_select=1),
    3: Workload(3, "wan1.3b-warmup", "bf16", 12, 128, 30, warmup_chunks(), lam=1e-2, k_select=15),
    4: Workload(4, "wan14b-warmup", "bf16", 40, 128, 40, warmup_chunks(), lam=1e-2, k_select=20),
    5: Workload(5, "wan1.3b-long", "bf16", 12, 128, 1,
                (Chunk(sink=(0, 3), cur=(63, 66), hist=(3, 63)),), lam=1e-2, k_select=1),
}


def rng_for(cfg: int, layer: int, stream: int, base: Optional[int] = None) -> np.random.Generator:
    b = SEED_BASE if base is None else base
    return np.random.default_rng(np.random.SeedSequence([b, cfg, layer, stream]))


# ----------------------------------------------------------------------------------------------
# Attention inputs
# ----------------------------------------------------------------------------------------------

def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def ar1_key_frames(rng: np.random.Generator, n_frames: int, n_heads: int, head_dim: int,
                   rho: float = AR_RHO, frame_tokens: int = FRAME_TOKENS) -> np.ndarray:
    """Keys of all frames [n_frames * frame_tokens, H, d_h] as one AR(1) chain per (position, head, channel)."""
    out = np.empty((n_frames, frame_tokens, n_heads, head_dim), dtype=np.float32)
    s = np.float32(np.sqrt(1.0 - rho * rho))
    out[0] = _normal(rng, (frame_tokens, n_heads, head_dim))
    for t in range(1, n_frames):
        out[t] = np.float32(rho) * out[t - 1] + s * _normal(rng, (frame_tokens, n_heads, head_dim))
    return out.reshape(n_frames * frame_tokens, n_heads, head_dim)


class LayerCache:
    """Keys and values of every latent frame of one layer (float32 holding input-precision values)."""

    def __init__(self, wl: Workload, layer: int, base: Optional[int] = None):
        self.wl = wl
        self.layer = layer
        self.base = base
        nf = wl.n_frames()
        rk = rng_for(wl.cfg, layer, STREAM_K, base)
        rv = rng_for(wl.cfg, layer, STREAM_V, base)
        k = ar1_key_frames(rk, nf, wl.n_heads, wl.head_dim)
        v = _normal(rv, (nf * FRAME_TOKENS, wl.n_heads, wl.head_dim))
        if wl.dtype == "bf16":
            k = round_bf16(k)
            v = round_bf16(v)
        self.k = k
        self.v = v

    def frames(self, r: tuple):
        a, b = r[0] * FRAME_TOKENS, r[1] * FRAME_TOKENS
        return self.k[a:b], self.v[a:b]


def attention_inputs(cfg: int, layer: int = 0, chunk: int = 0, base: Optional[int] = None,
                     cache: Optional[LayerCache] = None) -> Dict[str, object]:
    """Q and the three K/V segments of one (layer, chunk) of a workload.

    Returns float32 arrays holding the exact input values ("q", "sink_k", "sink_v", "cur_k",
    "cur_v", "hist_k", "hist_v"), plus "scale" and "dtype".
    """
    wl = CONFIGS[cfg]
    H, dh = wl.n_heads, wl.head_dim
    if wl.iid_tokens is not None:
        n_q, n_s, n_c, n_h = wl.iid_tokens
        rk = rng_for(cfg, layer, STREAM_K, base)
        rv = rng_for(cfg, layer, STREAM_V, base)
        rq = rng_for(cfg, layer, STREAM_Q0 + chunk, base)
        n_all = n_s + n_c + n_h
        k = _normal(rk, (n_all, H, dh))
        v = _normal(rv, (n_all, H, dh))
        q = _normal(rq, (n_q, H, dh))
        if wl.dtype == "bf16":
            k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
        segs = {"sink": (0, n_s), "cur": (n_s, n_s + n_c), "hist": (n_s + n_c, n_all)}
        out = {"q": q}
        for name, (a, b) in segs.items():
            out[name + "_k"] = k[a:b]
            out[name + "_v"] = v[a:b]
    else:
        if cache is None:
            cache = LayerCache(wl, layer, base)
        ch = wl.chunks[chunk]
        n_q = (ch.cur[1] - ch.cur[0]) * FRAME_TOKENS
        rq = rng_for(cfg, layer, STREAM_Q0 + chunk, base)
        q = _normal(rq, (n_q, H, dh))
        if wl.dtype == "bf16":
            q = round_bf16(q)
        out = {"q": q}
        for name in ("sink", "cur", "hist"):
            kk, vv = cache.frames(getattr(ch, name))
            out[name + "_k"] = kk
            out[name + "_v"] = vv
    out["scale"] = wl.scale
    out["dtype"] = wl.dtype
    return out


def attention_case(seed: int, n_heads: int, head_dim: int, n_q: int, n_sink: int, n_cur: int,
                   n_hist: int, dtype: str = "bf16", rho: Optional[float] = None,
                   scale: Optional[float] = None) -> Dict[str, object]:
    """A free-form attention case (for ragged and edge-case tests).

    Keys are iid N(0,1), or, with `rho`, one AR(1) chain over the token index in the order
    sink, history, current (temporal order of the cache).
    """
    rng = np.random.default_rng(np.random.SeedSequence([SEED_BASE, 1000, seed]))
    n_all = n_sink + n_cur + n_hist
    if rho is None:
        k = _normal(rng, (n_all, n_heads, head_dim))
    else:
        k = np.empty((n_all, n_heads, head_dim), dtype=np.float32)
        s = np.float32(np.sqrt(1.0 - rho * rho))
        z = _normal(rng, (n_all, n_heads, head_dim))
        prev = None
        for t in range(n_all):
            prev = z[t] if prev is None else np.float32(rho) * prev + s * z[t]
            k[t] = prev
        # temporal order sink, history, current -> storage order sink, current, history
        k = np.concatenate([k[:n_sink], k[n_sink + n_hist:], k[n_sink:n_sink + n_hist]], axis=0)
    v = _normal(rng, (n_all, n_heads, head_dim))
    q = _normal(rng, (n_q, n_heads, head_dim))
    if dtype == "bf16":
        k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
    segs = {"sink": (0, n_sink), "cur": (n_sink, n_sink + n_cur), "hist": (n_sink + n_cur, n_all)}
    out: Dict[str, object] = {"q": q}
    for name, (a, b) in segs.items():
        out[name + "_k"] = k[a:b]
        out[name + "_v"] = v[a:b]
    out["scale"] = (1.0 / float(np.sqrt(head_dim))) if scale is None else float(scale)
    out["dtype"] = dtype
    return out


def csr_from_labels(labels) -> Tuple[np.ndarray, np.ndarray]:
    """Groups given as one label per token (labels 0 .. G-1, each used) -> (offsets [G+1] int32,
    members [n] int32): group g holds the tokens with label g in increasing token order."""
    lab = np.asarray(labels, dtype=np.int64)
    n_groups = int(lab.max()) + 1 if lab.size else 0
    counts = np.bincount(lab, minlength=n_groups)
    offsets = np.zeros(n_groups + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    members = np.argsort(lab, kind="stable").astype(np.int32)
    return offsets, members


def static_history_case(seed: int, n_heads: int, head_dim: int, n_q: int, n_sink: int, n_cur: int,
                        n_frames: int, frame_tokens: int, static_frac: float, dtype: str = "bf16",
                        scale: Optional[float] = None) -> Dict[str, object]:
    """An attention case whose history holds exact duplicate keys (video with a static region).

    The history is n_frames frames of frame_tokens tokens. A fixed random subset of
    round(static_frac * frame_tokens) token positions is static: its keys are the same in every
    frame; its values still differ per frame. All other keys, all values and the queries are iid
    N(0,1). Returns the case dict of `attention_case` plus "hist_labels" [n_hist] (one label per
    history token: static position p -> p's rank among the static positions, other tokens ->
    consecutive labels after those) and "hist_groups" = csr_from_labels(hist_labels).
    """
    rng = np.random.default_rng(np.random.SeedSequence([SEED_BASE, 1100, seed]))
    n_hist = n_frames * frame_tokens
    n_static = int(round(static_frac * frame_tokens))
    static_pos = np.sort(rng.choice(frame_tokens, size=n_static, replace=False))
    is_static = np.zeros(frame_tokens, dtype=bool)
    is_static[static_pos] = True
    rank = np.cumsum(is_static) - 1
    static_keys = _normal(rng, (n_static, n_heads, head_dim))
    hist_k = _normal(rng, (n_hist, n_heads, head_dim))
    labels = np.empty(n_hist, dtype=np.int64)
    nxt = n_static
    for f in range(n_frames):
        for p in range(frame_tokens):
            t = f * frame_tokens + p
            if is_static[p]:
                hist_k[t] = static_keys[rank[p]]
                labels[t] = rank[p]
            else:
                labels[t] = nxt
                nxt += 1
    sink_k = _normal(rng, (n_sink, n_heads, head_dim))
    cur_k = _normal(rng, (n_cur, n_heads, head_dim))
    v = _normal(rng, (n_sink + n_cur + n_hist, n_heads, head_dim))
    q = _normal(rng, (n_q, n_heads, head_dim))
    if dtype == "bf16":
        sink_k, cur_k, hist_k, v, q = (round_bf16(x) for x in (sink_k, cur_k, hist_k, v, q))
    out: Dict[str, object] = {"q": q, "sink_k": sink_k, "cur_k": cur_k, "hist_k": hist_k,
                              "sink_v": v[:n_sink], "cur_v": v[n_sink:n_sink + n_cur],
                              "hist_v": v[n_sink + n_cur:]}
    out["scale"] = (1.0 / float(np.sqrt(head_dim))) if scale is None else float(scale)
    out["dtype"] = dtype
    out["hist_labels"] = labels
    out["hist_groups"] = csr_from_labels(labels)
    return out


# ----------------------------------------------------------------------------------------------
# Layer-absorb inputs
# ----------------------------------------------------------------------------------------------

def weight(cfg: int, layer: int, base: Optional[int] = None, d: Optional[int] = None) -> np.ndarray:
    """Output-projection weight W [d, d] ~ N(0, 1/d), float32, y = A @ W."""
    wl = CONFIGS.get(cfg)
    dd = d if d is not None else wl.d
    rng = rng_for(cfg, layer, STREAM_W, base)
    return (_normal(rng, (dd, dd)) * np.float32(1.0 / np.sqrt(dd))).astype(np.float32)


def absorb_rows(cfg: int, layer: int, chunk: int, base: Optional[int] = None,
                d: Optional[int] = None, n_rows: Optional[int] = None,
                dtype: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Synthetic (A_loc, A_full) rows of one (layer, warmup chunk), shaped like attention outputs.

    Attention outputs of N(0,1) values over n keys have entries of size about n**-0.5 and a
    spread of column energies; these rows imitate that without computing attention:
      A_loc  = 0.02 * Z1 * s            with column scales s_j = exp(-2.5 * u_j), u_j ~ U(0,1)
      A_full = A_loc                    for chunks with an empty history (chunks 0 and 1)
      A_full = (1-b) A_loc + b * (0.6 A_loc[:, perm] * r + 0.02 * Z2 * s)   otherwise,
    where perm is a fixed column permutation, r a per-column factor in [0.5, 1.5] and
    b = 0.1 + 0.5 * t_layer with t_layer ~ U(0,1) drawn per layer, so layers differ in how much
    history they miss. Values are rounded to the workload's dtype; rows are independent per chunk.
    """
    wl = CONFIGS[cfg]
    dd = d if d is not None else wl.d
    dt = dtype if dtype is not None else wl.dtype
    if n_rows is None:
        n_rows = wl.segment_sizes(chunk)["n_q"]
    has_hist = wl.iid_tokens is not None or wl.segment_sizes(chunk)["n_hist"] > 0
    lay = rng_for(cfg, layer, STREAM_ABSORB0 - 1, base)   # per-layer constants
    s = np.exp(-2.5 * lay.random(dd)).astype(np.float32)
    perm = lay.permutation(dd)
    r = (0.5 + lay.random(dd)).astype(np.float32)
    b = np.float32(0.1 + 0.5 * lay.random())
    rng = rng_for(cfg, layer, STREAM_ABSORB0 + chunk, base)
    a_loc = np.float32(0.02) * _normal(rng, (n_rows, dd)) * s
    if dt == "bf16":
        a_loc = round_bf16(a_loc)
    if has_hist:
        mix = np.float32(0.6) * a_loc[:, perm] * r + np.float32(0.02) * _normal(rng, (n_rows, dd)) * s
        a_full = (np.float32(1.0) - b) * a_loc + b * mix
        if dt == "bf16":
            a_full = round_bf16(a_full)
    else:
        a_full = a_loc.copy()
    return {"a_loc": np.ascontiguousarray(a_loc, dtype=np.float32),
            "a_full": np.ascontiguousarray(a_full, dtype=np.float32)}


def config_list() -> List[int]:
    return sorted(CONFIGS)
