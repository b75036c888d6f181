"""Python binding of libispa.so, the gfx950 library for ISPA's dual-stream attention and Layer Absorb.

The functions below carry the names of the C ABI (include/ispa.h) and only marshal arguments: torch
tensors become device pointers, sizes and strides, and the call is enqueued on the current HIP
stream (or the one given). Every step of the computation runs in the library's HIP kernels; there is
no fallback. If libispa.so is missing, importing the functions raises.

Build the library with ``python -m kv_cache_attention_split_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

from ._abi import (ISPA_BF16, ISPA_F32, ISPA_OK, IspaError, KVBias, KVSegment, lib, lib_path,  # noqa: F401
                   status_string)

__all__ = [
    "ispa_attn_dual", "ispa_attn_dual_balanced", "ispa_attn_dual_balanced_workspace", "ispa_attn_dual_biased", "ispa_kv_merge", "ispa_future_scores",
    "ispa_future_scores_workspace", "ispa_future_scores_noalloc", "ispa_fp8_head_scales", "ispa_fp8_quantize", "ispa_attn_dual_fp8",
    "ispa_attn_dual_fp8_pv",
    "ispa_absorb_accumulate", "ispa_absorb_accumulate_batched", "ispa_absorb_accumulate_fp8", "ispa_absorb_accumulate_workspace",
    "ispa_absorb_solve", "ispa_absorb_solve_workspace", "ispa_absorb_solve_eps",
    "ispa_absorb_solve_eps_workspace", "ispa_layer_error",
    "ispa_layer_error_workspace", "ispa_rank_layers", "ispa_apply_delta", "ispa_project",
    "ispa_kv_plan", "ispa_status_string", "ispa_version",
    "IspaError", "lib_path",
]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ISPA_BF16
    if t.dtype == torch.float32:
        return ISPA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_handle(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _check(status: int, what: str) -> None:
    if status != ISPA_OK:
        raise IspaError(status, f"{what}: {status_string(status)}")


def _seg(k, v, n_heads: int, head_dim: int) -> KVSegment:
    if k is None or k.shape[0] == 0:
        return KVSegment(None, None, 0, n_heads * head_dim)
    for t in (k, v):
        if t.dim() != 3 or t.shape[1] != n_heads or t.shape[2] != head_dim:
            raise ValueError(f"K/V segment must be [n, {n_heads}, {head_dim}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != head_dim:
            raise ValueError("K/V segment rows must be contiguous over (H, d_h)")
    if k.shape[0] != v.shape[0] or k.stride(0) != v.stride(0):
        raise ValueError("K and V of a segment must have the same length and row stride")
    return KVSegment(k.data_ptr(), v.data_ptr(), int(k.shape[0]), int(k.stride(0)))


def ispa_attn_dual(q, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v, softmax_scale: float,
                   a_loc, a_full=None, lse_loc=None, lse_hist=None, lse_full=None, stream=None) -> None:
    """Dual-stream attention (see ispa_attn_dual in include/ispa.h).

    q: [n_q, H, d_h]; *_k/*_v: [n, H, d_h] (a segment may be None or have n = 0); a_loc / a_full:
    [n_q, H*d_h] preallocated outputs of q's dtype; lse_*: [H, n_q] float32 outputs or None.
    """
    n_q, H, dh = (int(x) for x in q.shape)
    if q.stride(2) != 1 or q.stride(1) != dh:
        raise ValueError("q rows must be contiguous over (H, d_h)")
    for o in (a_loc, a_full):
        if o is not None and (tuple(o.shape) != (n_q, H * dh) or not o.is_contiguous() or o.dtype != q.dtype):
            raise ValueError("outputs must be contiguous [n_q, H*d_h] of q's dtype")
    torch = _torch()
    for o in (lse_loc, lse_hist, lse_full):
        if o is not None and (tuple(o.shape) != (H, n_q) or not o.is_contiguous() or o.dtype != torch.float32):
            raise ValueError("LSE outputs must be contiguous float32 [H, n_q]")
    st = lib().ispa_attn_dual(
        _dtype_code(q), H, dh, ctypes.c_float(softmax_scale), _ptr(q), n_q, int(q.stride(0)),
        _seg(sink_k, sink_v, H, dh), _seg(cur_k, cur_v, H, dh), _seg(hist_k, hist_v, H, dh),
        _ptr(a_loc), _ptr(a_full), _ptr(lse_loc), _ptr(lse_hist), _ptr(lse_full), _stream_handle(stream))
    _check(st, "ispa_attn_dual")


def _seg_len(k) -> int:
    return 0 if k is None else int(k.shape[0])


def ispa_attn_dual_balanced_workspace(q, n_local_keys: int, n_hist_keys: int) -> int:
    """Scratch bytes for ispa_attn_dual_balanced with queries like `q` ([n_q, H, d_h]) on the current
    device (0: the plain schedule is used and no scratch is needed)."""
    n_q, H, dh = (int(x) for x in q.shape)
    return int(lib().ispa_attn_dual_balanced_workspace(_dtype_code(q), H, dh, n_q, int(n_local_keys),
                                                       int(n_hist_keys)))


def ispa_attn_dual_balanced(q, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v, softmax_scale: float,
                            a_loc, a_full=None, lse_loc=None, lse_hist=None, lse_full=None, ws=None,
                            stream=None) -> None:
    """ispa_attn_dual with the balanced schedule over the compute units (see include/ispa.h). ws: uint8
    device scratch of ispa_attn_dual_balanced_workspace bytes (allocated for the call if None)."""
    n_q, H, dh = (int(x) for x in q.shape)
    if q.stride(2) != 1 or q.stride(1) != dh:
        raise ValueError("q rows must be contiguous over (H, d_h)")
    for o in (a_loc, a_full):
        if o is not None and (tuple(o.shape) != (n_q, H * dh) or not o.is_contiguous() or o.dtype != q.dtype):
            raise ValueError("outputs must be contiguous [n_q, H*d_h] of q's dtype")
    torch = _torch()
    for o in (lse_loc, lse_hist, lse_full):
        if o is not None and (tuple(o.shape) != (H, n_q) or not o.is_contiguous() or o.dtype != torch.float32):
            raise ValueError("LSE outputs must be contiguous float32 [H, n_q]")
    n_hist = _seg_len(hist_k) if a_full is not None else 0
    need = ispa_attn_dual_balanced_workspace(q, _seg_len(sink_k) + _seg_len(cur_k), n_hist)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None and (ws.dtype != torch.uint8 or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous uint8 tensor")
    st = lib().ispa_attn_dual_balanced(
        _dtype_code(q), H, dh, ctypes.c_float(softmax_scale), _ptr(q), n_q, int(q.stride(0)),
        _seg(sink_k, sink_v, H, dh), _seg(cur_k, cur_v, H, dh), _seg(hist_k, hist_v, H, dh),
        _ptr(a_loc), _ptr(a_full), _ptr(lse_loc), _ptr(lse_hist), _ptr(lse_full), _ptr(ws),
        0 if ws is None else int(ws.numel()), _stream_handle(stream))
    _check(st, "ispa_attn_dual_balanced")


def _bias_arg(t, n: int, n_heads: int):
    """(pointer, head stride) of a segment bias: None, [n] (all heads) or [H, stride >= n] fp32."""
    if t is None or n == 0:
        return None, None
    torch = _torch()
    if t.dtype != torch.float32 or t.stride(-1) != 1:
        raise ValueError("a bias must be float32 with unit stride over the keys")
    if t.dim() == 1:
        if t.shape[0] != n:
            raise ValueError(f"bias of {t.shape[0]} keys for a segment of {n}")
        return _ptr(t), 0
    if t.dim() != 2 or t.shape[0] != n_heads or t.shape[1] != n:
        raise ValueError(f"a per-head bias must be [{n_heads}, {n}]")
    return _ptr(t), int(t.stride(0))


def ispa_attn_dual_biased(q, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v, softmax_scale: float,
                          a_loc, a_full=None, lse_loc=None, lse_hist=None, lse_full=None,
                          sink_bias=None, cur_bias=None, hist_bias=None, stream=None) -> None:
    """Dual-stream attention with a per-key additive logit bias (see ispa_attn_dual_biased in
    include/ispa.h). Each *_bias is None, float32 [n] (shared by the heads) or [H, n] (a view with
    unit stride over the keys)."""
    n_q, H, dh = (int(x) for x in q.shape)
    if q.stride(2) != 1 or q.stride(1) != dh:
        raise ValueError("q rows must be contiguous over (H, d_h)")
    for o in (a_loc, a_full):
        if o is not None and (tuple(o.shape) != (n_q, H * dh) or not o.is_contiguous() or o.dtype != q.dtype):
            raise ValueError("outputs must be contiguous [n_q, H*d_h] of q's dtype")
    torch = _torch()
    for o in (lse_loc, lse_hist, lse_full):
        if o is not None and (tuple(o.shape) != (H, n_q) or not o.is_contiguous() or o.dtype != torch.float32):
            raise ValueError("LSE outputs must be contiguous float32 [H, n_q]")
    segs = [_seg(sink_k, sink_v, H, dh), _seg(cur_k, cur_v, H, dh), _seg(hist_k, hist_v, H, dh)]
    args = [_bias_arg(b, int(sg.n), H) for b, sg in zip((sink_bias, cur_bias, hist_bias), segs)]
    bias = KVBias(args[0][0], args[1][0], args[2][0], args[0][1] or 0, args[1][1] or 0, args[2][1] or 0)
    st = lib().ispa_attn_dual_biased(
        _dtype_code(q), H, dh, ctypes.c_float(softmax_scale), _ptr(q), n_q, int(q.stride(0)),
        segs[0], segs[1], segs[2], ctypes.byref(bias),
        _ptr(a_loc), _ptr(a_full), _ptr(lse_loc), _ptr(lse_hist), _ptr(lse_full), _stream_handle(stream))
    _check(st, "ispa_attn_dual_biased")


def ispa_kv_merge(k, v, offsets, members, k_out, v_out, bias_out=None, stream=None) -> None:
    """TempCache merge of one segment (see ispa_kv_merge in include/ispa.h): k, v [n, H, d_h];
    offsets int32 [G+1], members int32 [offsets[G]] on the device; k_out, v_out [G, H, d_h] of k's
    dtype; bias_out float32 [G] or None."""
    n = int(k.shape[0])
    width = int(k.shape[1] * k.shape[2])
    n_groups = int(offsets.shape[0]) - 1
    torch = _torch()
    for t in (k, v):
        if t.dtype != k.dtype or tuple(t.shape[1:]) != tuple(k.shape[1:]) or t.stride(2) != 1 or \
                t.stride(1) != k.shape[2] or t.stride(0) != k.stride(0) or t.shape[0] != n:
            raise ValueError("k and v must be matching [n, H, d_h] with contiguous rows")
    for t in (k_out, v_out):
        if t.dtype != k.dtype or tuple(t.shape) != (n_groups,) + tuple(k.shape[1:]) or t.stride(2) != 1 or \
                t.stride(1) != k.shape[2] or t.stride(0) != k_out.stride(0):
            raise ValueError("k_out and v_out must be [G, H, d_h] of k's dtype with contiguous rows")
    for t in (offsets, members):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("offsets and members must be contiguous int32")
    if bias_out is not None and (bias_out.dtype != torch.float32 or tuple(bias_out.shape) != (n_groups,)):
        raise ValueError("bias_out must be float32 [G]")
    st = lib().ispa_kv_merge(
        _dtype_code(k), width, _ptr(k), _ptr(v), n, int(k.stride(0)) if n else width, _ptr(offsets),
        _ptr(members), n_groups, _ptr(k_out), _ptr(v_out), int(k_out.stride(0)) if n_groups else width,
        _ptr(bias_out), _stream_handle(stream))
    _check(st, "ispa_kv_merge")


def _rows3(x):
    if x.dim() != 3 or x.stride(2) != 1 or x.stride(1) != x.shape[2]:
        raise ValueError("rows must be [n, H, d_h], contiguous over (H, d_h)")
    return int(x.shape[0]), int(x.shape[1]), int(x.shape[2]), int(x.stride(0))


def ispa_fp8_head_scales(x, scales, stream=None) -> None:
    """scales[h] = max |x[:, h, :]| / 448 (1 for an all-zero head); x bf16/fp32 [n, H, d_h]."""
    n, H, dh, st = _rows3(x)
    if tuple(scales.shape) != (H,) or scales.dtype != _torch().float32:
        raise ValueError("scales must be float32 [H]")
    s = lib().ispa_fp8_head_scales(_dtype_code(x), _ptr(x), n, H, dh, st, _ptr(scales), _stream_handle(stream))
    _check(s, "ispa_fp8_head_scales")


def ispa_fp8_quantize(x, scales, out, stream=None) -> None:
    """out = e4m3 codes of x / scales (per head), uint8 [n, H, d_h] with contiguous rows."""
    n, H, dh, st = _rows3(x)
    torch = _torch()
    if out.dtype != torch.uint8 or tuple(out.shape) != (n, H, dh) or out.stride(2) != 1 or out.stride(1) != dh:
        raise ValueError("out must be uint8 [n, H, d_h] with contiguous rows")
    s = lib().ispa_fp8_quantize(_dtype_code(x), _ptr(x), n, H, dh, st, _ptr(scales), _ptr(out),
                                int(out.stride(0)) if n else H * dh, _stream_handle(stream))
    _check(s, "ispa_fp8_quantize")


def _seg_fp8(k, v, n_heads: int, head_dim: int, v_fp8: bool = False) -> KVSegment:
    if k is None or k.shape[0] == 0:
        return KVSegment(None, None, 0, n_heads * head_dim)
    for t in (k, v):
        if t.dim() != 3 or t.shape[1] != n_heads or t.shape[2] != head_dim or t.stride(2) != 1 or \
                t.stride(1) != head_dim:
            raise ValueError("K/V segment must be [n, H, d_h] with contiguous rows")
    torch = _torch()
    if k.dtype != torch.uint8 or v.dtype != (torch.uint8 if v_fp8 else torch.bfloat16):
        raise ValueError("K must be uint8 e4m3 codes and V " + ("uint8 e4m3 codes" if v_fp8 else "bfloat16"))
    if k.shape[0] != v.shape[0] or k.stride(0) != v.stride(0):
        raise ValueError("K and V of a segment must have the same rows and row stride")
    return KVSegment(_ptr(k), _ptr(v), int(k.shape[0]), int(k.stride(0)))


def ispa_attn_dual_fp8(q, q_scale, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v, k_scale, softmax_scale: float,
                       a_loc, a_full=None, lse_loc=None, lse_hist=None, lse_full=None, stream=None) -> None:
    """Dual-stream attention with e4m3 q and keys (uint8 codes, float32 per-head scales) and bf16 values
    (see ispa_attn_dual_fp8 in include/ispa.h)."""
    n_q, H, dh = (int(x) for x in q.shape)
    if q.stride(2) != 1 or q.stride(1) != dh:
        raise ValueError("q rows must be contiguous over (H, d_h)")
    st = lib().ispa_attn_dual_fp8(
        H, dh, ctypes.c_float(softmax_scale), _ptr(q), n_q, int(q.stride(0)), _ptr(q_scale),
        _seg_fp8(sink_k, sink_v, H, dh), _seg_fp8(cur_k, cur_v, H, dh), _seg_fp8(hist_k, hist_v, H, dh),
        _ptr(k_scale), _ptr(a_loc), _ptr(a_full), _ptr(lse_loc), _ptr(lse_hist), _ptr(lse_full),
        _stream_handle(stream))
    _check(st, "ispa_attn_dual_fp8")


def ispa_attn_dual_fp8_pv(q, q_scale, sink_k, sink_v, cur_k, cur_v, hist_k, hist_v, k_scale, v_scale,
                          softmax_scale: float, a_loc, a_full=None, lse_loc=None, lse_hist=None, lse_full=None,
                          stream=None) -> None:
    """Dual-stream attention with e4m3 q, keys and values (uint8 codes, float32 per-head scales) and the
    value product in FP8 (see ispa_attn_dual_fp8_pv in include/ispa.h)."""
    n_q, H, dh = (int(x) for x in q.shape)
    if q.stride(2) != 1 or q.stride(1) != dh:
        raise ValueError("q rows must be contiguous over (H, d_h)")
    st = lib().ispa_attn_dual_fp8_pv(
        H, dh, ctypes.c_float(softmax_scale), _ptr(q), n_q, int(q.stride(0)), _ptr(q_scale),
        _seg_fp8(sink_k, sink_v, H, dh, True), _seg_fp8(cur_k, cur_v, H, dh, True),
        _seg_fp8(hist_k, hist_v, H, dh, True), _ptr(k_scale), _ptr(v_scale), _ptr(a_loc), _ptr(a_full),
        _ptr(lse_loc), _ptr(lse_hist), _ptr(lse_full), _stream_handle(stream))
    _check(st, "ispa_attn_dual_fp8_pv")


def ispa_future_scores_workspace(n_heads: int, n_p: int) -> int:
    return int(lib().ispa_future_scores_workspace(int(n_heads), int(n_p)))


def _key_seg(k, n_heads: int, head_dim: int) -> KVSegment:
    if k is None or k.shape[0] == 0:
        return KVSegment(None, None, 0, n_heads * head_dim)
    if k.dim() != 3 or k.shape[1] != n_heads or k.shape[2] != head_dim:
        raise ValueError(f"keys must be [n, {n_heads}, {head_dim}], got {tuple(k.shape)}")
    if k.stride(2) != 1 or k.stride(1) != head_dim:
        raise ValueError("key rows must be contiguous over (H, d_h)")
    return KVSegment(_ptr(k), None, int(k.shape[0]), int(k.stride(0)))


def ispa_future_scores(q_proxy, sink_k, cur_k, hist_k, softmax_scale: float, scores, ws=None,
                       lam: float = 1.0, hist_token_score=None, token_score=None, stream=None) -> None:
    """Future-query importance of the cached keys (see ispa_future_scores in include/ispa.h).

    q_proxy: bf16 [n_p, H, d_h]; *_k: bf16 [n, H, d_h] or None; scores: float32 [H, >= total keys]
    (a view with unit stride over the keys); token_score / hist_token_score: float32 [total] or None.
    ws: device scratch of ispa_future_scores_workspace(H, n_p) bytes (allocated for the call if None).
    """
    n_p, H, dh = (int(x) for x in q_proxy.shape)
    if q_proxy.stride(2) != 1 or q_proxy.stride(1) != dh:
        raise ValueError("proxy rows must be contiguous over (H, d_h)")
    torch = _torch()
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[0] != H or scores.stride(1) != 1:
        raise ValueError("scores must be float32 [H, n] with unit stride over the keys")
    for t in (hist_token_score, token_score):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("token scores must be contiguous float32")
    if ws is None:
        ws = torch.empty(max(1, ispa_future_scores_workspace(H, n_p)), dtype=torch.uint8, device=q_proxy.device)
    st = lib().ispa_future_scores(
        _dtype_code(q_proxy), H, dh, ctypes.c_float(softmax_scale), _ptr(q_proxy), n_p, int(q_proxy.stride(0)),
        _key_seg(sink_k, H, dh), _key_seg(cur_k, H, dh), _key_seg(hist_k, H, dh), _ptr(scores),
        int(scores.stride(0)), ctypes.c_float(lam), _ptr(hist_token_score), _ptr(token_score), _ptr(ws),
        int(ws.numel() * ws.element_size()), _stream_handle(stream))
    _check(st, "ispa_future_scores")


def ispa_future_scores_noalloc(q_proxy, sink_k, cur_k, hist_k, softmax_scale: float, scores, lam: float = 1.0,
                               hist_token_score=None, token_score=None, stream=None) -> None:
    """ispa_future_scores with the library's own per-GPU scratch instead of a workspace (see
    ispa_future_scores_noalloc in include/ispa.h): allocates nothing; calls that overlap on one GPU race."""
    n_p, H, dh = (int(x) for x in q_proxy.shape)
    if q_proxy.stride(2) != 1 or q_proxy.stride(1) != dh:
        raise ValueError("proxy rows must be contiguous over (H, d_h)")
    torch = _torch()
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[0] != H or scores.stride(1) != 1:
        raise ValueError("scores must be float32 [H, n] with unit stride over the keys")
    for t in (hist_token_score, token_score):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("token scores must be contiguous float32")
    st = lib().ispa_future_scores_noalloc(
        _dtype_code(q_proxy), H, dh, ctypes.c_float(softmax_scale), _ptr(q_proxy), n_p, int(q_proxy.stride(0)),
        _key_seg(sink_k, H, dh), _key_seg(cur_k, H, dh), _key_seg(hist_k, H, dh), _ptr(scores),
        int(scores.stride(0)), ctypes.c_float(lam), _ptr(hist_token_score), _ptr(token_score),
        _stream_handle(stream))
    _check(st, "ispa_future_scores_noalloc")


def ispa_absorb_accumulate_workspace(n_rows: int, d: int) -> int:
    return int(lib().ispa_absorb_accumulate_workspace(int(n_rows), int(d)))


def ispa_absorb_accumulate(a_loc, a_full, G, X, F=None, ws=None, stream=None) -> None:
    """G += A_loc^T A_loc, X += A_loc^T A_full, F += A_full^T A_full (fp32 [d, d], in place)."""
    n, d = (int(x) for x in a_loc.shape)
    if tuple(a_full.shape) != (n, d) or a_full.dtype != a_loc.dtype:
        raise ValueError("a_loc and a_full must match")
    for t, what in ((a_loc, "a_loc"), (a_full, "a_full")):
        _device_tensor(t, what)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    _square_list([G, X] + ([F] if F is not None else []), d, 3 if F is not None else 2, "statistic")
    ws_ptr, ws_bytes = _workspace(ws)
    st = lib().ispa_absorb_accumulate(
        _dtype_code(a_loc), n, d, _ptr(a_loc), _ptr(a_full), _ptr(G), _ptr(X), _ptr(F),
        ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "ispa_absorb_accumulate")


def ispa_absorb_accumulate_batched(a_loc: Sequence, a_full: Sequence, G: Sequence, X: Sequence,
                                   F: Optional[Sequence] = None, stream=None) -> None:
    """For each layer l: G[l] += A_loc[l]^T A_loc[l], X[l] += A_loc[l]^T A_full[l], F[l] += A_full[l]^T A_full[l]
    (lists of [n, d] rows of one dtype and [d, d] fp32 sums; every layer the same n and d)."""
    batch = len(a_loc)
    if batch == 0:
        return
    n, d = (int(x) for x in a_loc[0].shape)
    if len(a_full) != batch:
        raise ValueError("a_loc and a_full must have one entry per layer")
    for t, what in [(t, "a_loc") for t in a_loc] + [(t, "a_full") for t in a_full]:
        if tuple(t.shape) != (n, d) or t.dtype != a_loc[0].dtype or not t.is_contiguous():
            raise ValueError(f"every {what} entry must be a contiguous [{n}, {d}] tensor of one dtype")
        _device_tensor(t, what)
    ptrs = [_square_list(m, d, batch, name) for m, name in ((G, "G"), (X, "X"))]
    fp = _square_list(F, d, batch, "F") if F is not None else None
    st = lib().ispa_absorb_accumulate_batched(
        _dtype_code(a_loc[0]), n, d, batch, _ptr_array(a_loc), _ptr_array(a_full), ptrs[0], ptrs[1], fp,
        _stream_handle(stream))
    _check(st, "ispa_absorb_accumulate_batched")


def ispa_absorb_accumulate_fp8(a_loc, s_loc, a_full, s_full, head_dim: int, G, X, F=None, stream=None) -> None:
    """FP8 statistics: a_loc, a_full uint8 e4m3 codes [n, d] (contiguous), s_loc, s_full float32 per-head
    scales [d / head_dim]; G, X, F as for ispa_absorb_accumulate."""
    n, d = (int(x) for x in a_loc.shape)
    torch = _torch()
    if tuple(a_full.shape) != (n, d):
        raise ValueError("a_loc and a_full must match")
    for t, what in ((a_loc, "a_loc"), (a_full, "a_full")):
        _device_tensor(t, what)
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("FP8 rows must be contiguous uint8 (e4m3 codes)")
    if head_dim <= 0 or d % head_dim != 0:
        raise ValueError("d must be a multiple of head_dim")
    for t, what in ((s_loc, "s_loc"), (s_full, "s_full")):
        _vector(t, d // head_dim, torch.float32, what)
    _square_list([G, X] + ([F] if F is not None else []), d, 3 if F is not None else 2, "statistic")
    st = lib().ispa_absorb_accumulate_fp8(n, d, int(head_dim), _ptr(a_loc), _ptr(s_loc), _ptr(a_full), _ptr(s_full),
                                          _ptr(G), _ptr(X), _ptr(F), None, 0, _stream_handle(stream))
    _check(st, "ispa_absorb_accumulate_fp8")


def _ptr_array(ts: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        if not t.is_contiguous():
            raise ValueError("per-layer matrices must be contiguous")
        arr[i] = t.data_ptr()
    return arr


def _device_tensor(t, what: str) -> None:
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")


def _square_list(ts: Sequence, d: int, batch: int, what: str) -> ctypes.Array:
    """Device pointers of `batch` contiguous float32 [d, d] GPU matrices."""
    torch = _torch()
    if len(ts) != batch:
        raise ValueError(f"{what} must have one entry per layer ({batch}), got {len(ts)}")
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or tuple(t.shape) != (d, d) or \
                not t.is_contiguous():
            raise ValueError(f"every {what} entry must be a contiguous float32 [{d}, {d}] tensor")
        _device_tensor(t, what)
    return _ptr_array(ts)


def _vector(t, n: int, dtype, what: str, optional: bool = False) -> None:
    if t is None:
        if optional:
            return
        raise ValueError(f"{what} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != 1 or t.shape[0] < n or \
            not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {dtype} vector of at least {n} entries")
    _device_tensor(t, what)


def _workspace(ws):
    if ws is None:
        return None, 0
    _device_tensor(ws, "ws")
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")
    return _ptr(ws), int(ws.numel() * ws.element_size())


def ispa_absorb_solve_workspace(d: int, batch: int) -> int:
    return int(lib().ispa_absorb_solve_workspace(int(d), int(batch)))


def ispa_absorb_solve(G: Sequence, X: Sequence, W: Sequence, dW: Sequence, lam: float, info,
                      ws, w_is_linear_weight: bool = False, stream=None) -> None:
    """dW_l = (G_l + lam I)^-1 (X_l - G_l) W_l for each layer l (lists of [d, d] fp32 tensors)."""
    batch = len(G)
    d = int(G[0].shape[0]) if batch else 0
    torch = _torch()
    ptrs = [_square_list(m, d, batch, name) for m, name in ((G, "G"), (X, "X"), (W, "W"), (dW, "dW"))]
    if batch:
        _vector(info, batch, torch.int32, "info")
    ws_ptr, ws_bytes = _workspace(ws)
    st = lib().ispa_absorb_solve(
        d, batch, ctypes.c_float(lam), ptrs[0], ptrs[1], ptrs[2], 1 if w_is_linear_weight else 0, ptrs[3],
        _ptr(info), ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "ispa_absorb_solve")


def ispa_absorb_solve_eps_workspace(d: int, batch: int) -> int:
    return int(lib().ispa_absorb_solve_eps_workspace(int(d), int(batch)))


def ispa_absorb_solve_eps(G: Sequence, X: Sequence, F: Sequence, W: Sequence, dW: Sequence, lam: float, info, eps,
                          ref=None, ws=None, w_is_linear_weight: bool = False, stream=None) -> None:
    """dW as ispa_absorb_solve, plus eps_l = ||A_loc (W + dW) - A_full W||_F^2 at that optimum and
    ref_l = ||A_full W||_F^2 (float64 [batch]; eps is NaN where info is nonzero)."""
    batch = len(G)
    d = int(G[0].shape[0]) if batch else 0
    torch = _torch()
    ptrs = [_square_list(m, d, batch, name) for m, name in ((G, "G"), (X, "X"), (F, "F"), (W, "W"), (dW, "dW"))]
    if batch:
        _vector(info, batch, torch.int32, "info")
        _vector(eps, batch, torch.float64, "eps")
        _vector(ref, batch, torch.float64, "ref", optional=True)
    ws_ptr, ws_bytes = _workspace(ws)
    st = lib().ispa_absorb_solve_eps(
        d, batch, ctypes.c_float(lam), ptrs[0], ptrs[1], ptrs[2], ptrs[3], 1 if w_is_linear_weight else 0, ptrs[4],
        _ptr(info), _ptr(eps), _ptr(ref), ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "ispa_absorb_solve_eps")


def ispa_layer_error_workspace(d: int, batch: int) -> int:
    return int(lib().ispa_layer_error_workspace(int(d), int(batch)))


def ispa_layer_error(G: Sequence, X: Sequence, F: Sequence, W: Sequence, dW: Sequence, eps, ref=None,
                     ws=None, w_is_linear_weight: bool = False, stream=None) -> None:
    """eps_l = ||A_loc (W + dW) - A_full W||_F^2 from the statistics; ref_l = ||A_full W||_F^2."""
    batch = len(G)
    d = int(G[0].shape[0]) if batch else 0
    torch = _torch()
    ptrs = [_square_list(m, d, batch, name) for m, name in ((G, "G"), (X, "X"), (F, "F"), (W, "W"), (dW, "dW"))]
    if batch:
        _vector(eps, batch, torch.float64, "eps")
        _vector(ref, batch, torch.float64, "ref", optional=True)
    ws_ptr, ws_bytes = _workspace(ws)
    st = lib().ispa_layer_error(
        d, batch, ptrs[0], ptrs[1], ptrs[2], ptrs[3], 1 if w_is_linear_weight else 0, ptrs[4],
        _ptr(eps), _ptr(ref), ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "ispa_layer_error")


def ispa_rank_layers(eps: Sequence[float], k: int):
    """Host-only layer selection: (selected indices in ascending-eps order, 0/1 L-Layer flags)."""
    n = len(eps)
    e = (ctypes.c_double * max(1, n))(*[float(x) for x in eps])
    sel = (ctypes.c_int32 * max(1, k))()
    flag = (ctypes.c_uint8 * max(1, n))()
    st = lib().ispa_rank_layers(e, n, int(k), sel, flag)
    _check(st, "ispa_rank_layers")
    return [int(sel[i]) for i in range(k)], [int(flag[i]) for i in range(n)]


def ispa_apply_delta(W, dW, w_new, w_is_linear_weight: bool = False, stream=None) -> None:
    """w_new (bf16 [d_out, d_in]) = W + dW rounded to bf16; W, dW fp32 [d_in, d_out] (y = A W), or
    [d_out, d_in] with w_is_linear_weight."""
    r, c = (int(x) for x in W.shape)
    d_in, d_out = (c, r) if w_is_linear_weight else (r, c)
    if tuple(dW.shape) != (r, c) or tuple(w_new.shape) != (d_out, d_in):
        raise ValueError("ispa_apply_delta: W, dW must match and w_new must be [d_out, d_in]")
    st = lib().ispa_apply_delta(d_in, d_out, _ptr(W), _ptr(dW), int(bool(w_is_linear_weight)),
                                _ptr(w_new), _stream_handle(stream))
    _check(st, "ispa_apply_delta")


def ispa_project(a, w, y, stream=None) -> None:
    """y [n, d_out] = a [n, d_in] @ w^T, w [d_out, d_in]; bf16 tensors, rows may be strided."""
    n, d_in = (int(x) for x in a.shape)
    d_out = int(w.shape[0])
    if tuple(w.shape) != (d_out, d_in) or tuple(y.shape) != (n, d_out):
        raise ValueError("ispa_project: shapes must be a [n, d_in], w [d_out, d_in], y [n, d_out]")
    st = lib().ispa_project(n, d_in, d_out, _ptr(a), int(a.stride(0)) if n else d_in, _ptr(w), _ptr(y),
                            int(y.stride(0)) if n else d_out, _stream_handle(stream))
    _check(st, "ispa_project")


def ispa_kv_plan(is_l_layer: Sequence[int], n_sink: int, n_hist: int, n_cur: int):
    """Host-only: (history tokens kept per layer, evicted key/value tokens in total)."""
    n = len(is_l_layer)
    flags = (ctypes.c_uint8 * max(1, n))(*[1 if f else 0 for f in is_l_layer])
    kept = (ctypes.c_int64 * max(1, n))()
    ev = ctypes.c_int64(0)
    st = lib().ispa_kv_plan(n, flags, int(n_sink), int(n_hist), int(n_cur), kept, ctypes.byref(ev))
    _check(st, "ispa_kv_plan")
    return [int(kept[i]) for i in range(n)], int(ev.value)


def ispa_status_string(status: int) -> str:
    return status_string(status)


def ispa_version() -> int:
    return int(lib().ispa_version())
