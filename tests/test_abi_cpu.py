"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, rejects bad
arguments before touching the device, sizes its workspaces, and ranks layers like the oracle.

Only argument errors are exercised here: validation returns before any HIP call, so fake (aligned,
non-null) pointers are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import kv_cache_attention_split_amd as ispa
from kv_cache_attention_split_amd import _abi
from oracle import absorb as oab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ispa.h")

FAKE = 0x10000      # aligned, never dereferenced
FAKE2 = 0x20000
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ispa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _abi.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert "ispa_attn_dual" in names and "ispa_absorb_solve" in names and "ispa_layer_error" in names
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ispa_\w+)", out))
    for n in names:
        assert n in exported, n
        getattr(L, n)
    assert set(_abi.SIGNATURES) == set(names)


def test_status_strings_and_version(L):
    for code in (0, -1, -2, -3, -4):
        assert ispa.ispa_status_string(code).startswith("ISPA")
    assert ispa.ispa_version() >= 100


def seg(k=FAKE, v=FAKE2, n=16, stride=256):
    return _abi.KVSegment(k, v, n, stride)


def attn(L, dt=1, H=2, dh=128, scale=0.088, q=FAKE, n_q=32, q_stride=256, sink=None, cur=None,
         hist=None, a_loc=FAKE, a_full=FAKE2):
    sink = sink if sink is not None else seg()
    cur = cur if cur is not None else seg()
    hist = hist if hist is not None else seg()
    return L.ispa_attn_dual(dt, H, dh, ctypes.c_float(scale), q, n_q, q_stride, sink, cur, hist,
                            a_loc, a_full, None, None, None, None)


def test_attn_argument_errors(L):
    assert attn(L, dh=96) == _abi.ISPA_E_UNSUPPORTED
    assert attn(L, dt=7) == _abi.ISPA_E_UNSUPPORTED
    assert attn(L, H=0) == _abi.ISPA_E_ARG
    assert attn(L, scale=0.0) == _abi.ISPA_E_ARG
    assert attn(L, scale=float("nan")) == _abi.ISPA_E_ARG
    assert attn(L, n_q=-1) == _abi.ISPA_E_ARG
    # row strides of 2^23 elements or more are outside the kernels' 24-bit in-tile offsets
    assert attn(L, hist=seg(stride=1 << 23)) == _abi.ISPA_E_UNSUPPORTED
    assert attn(L, sink=seg(stride=(1 << 23) + 8)) == _abi.ISPA_E_UNSUPPORTED
    # empty local context (softmax over an empty set)
    assert attn(L, sink=seg(n=0), cur=seg(n=0)) == _abi.ISPA_E_ARG
    # misaligned pointers, short or misaligned strides
    assert attn(L, q=MISALIGNED) == _abi.ISPA_E_ARG
    assert attn(L, cur=seg(k=MISALIGNED)) == _abi.ISPA_E_ARG
    assert attn(L, q_stride=128) == _abi.ISPA_E_ARG
    assert attn(L, sink=seg(stride=260)) == _abi.ISPA_E_ARG     # not a multiple of 8
    assert attn(L, hist=seg(n=-3)) == _abi.ISPA_E_ARG
    assert attn(L, a_loc=0) == _abi.ISPA_E_ARG
    assert attn(L, a_loc=MISALIGNED) == _abi.ISPA_E_ARG
    # missing K/V of a non-empty segment
    assert attn(L, cur=seg(k=0)) == _abi.ISPA_E_ARG
    # n_q == 0 is a no-op that succeeds without touching the device
    assert attn(L, n_q=0) == _abi.ISPA_OK


def attn_b(L, bias, **kw):
    sink, cur, hist = kw.get("sink", seg()), kw.get("cur", seg()), kw.get("hist", seg())
    return L.ispa_attn_dual_biased(1, 2, 128, ctypes.c_float(0.088), FAKE, kw.get("n_q", 32), 256, sink, cur,
                                   hist, None if bias is None else ctypes.byref(bias), FAKE,
                                   kw.get("a_full", FAKE2), None, None, None, None)


def test_biased_attn_argument_errors(L):
    B = _abi.KVBias
    # the plain attention's checks come first
    assert L.ispa_attn_dual_biased(1, 2, 96, ctypes.c_float(0.088), FAKE, 32, 256, seg(), seg(), seg(),
                                   None, FAKE, FAKE2, None, None, None, None) == _abi.ISPA_E_UNSUPPORTED
    assert attn_b(L, B(FAKE, None, None, -1, 0, 0), n_q=0) == _abi.ISPA_E_ARG    # negative head stride
    assert attn_b(L, B(FAKE + 2, None, None, 0, 0, 0), n_q=0) == _abi.ISPA_E_ARG  # misaligned bias
    assert attn_b(L, B(None, FAKE, None, 0, 8, 0), n_q=0) == _abi.ISPA_E_ARG     # head stride < n (16)
    assert attn_b(L, B(None, None, FAKE, 0, 0, 15), n_q=0) == _abi.ISPA_E_ARG
    # valid layouts: shared (0) or a head stride >= n, per segment; NULL entries; a history bias is
    # ignored (not checked) when only the local branch is computed; strides of NULL entries are unread
    assert attn_b(L, None, n_q=0) == _abi.ISPA_OK
    assert attn_b(L, B(FAKE, FAKE, FAKE, 0, 0, 0), n_q=0) == _abi.ISPA_OK
    assert attn_b(L, B(FAKE, None, FAKE, 16, -5, 40), n_q=0) == _abi.ISPA_OK
    assert attn_b(L, B(None, None, FAKE + 2, 0, 0, 3), n_q=0, a_full=None) == _abi.ISPA_OK


def test_kv_merge_argument_errors(L):
    f = L.ispa_kv_merge
    ok = dict(dt=1, width=256, k=FAKE, v=FAKE2, n=10, in_stride=256, off=FAKE, mem=FAKE2, G=0, ko=FAKE,
              vo=FAKE2, out_stride=256, bias=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["dt"], a["width"], a["k"], a["v"], a["n"], a["in_stride"], a["off"], a["mem"], a["G"],
                 a["ko"], a["vo"], a["out_stride"], a["bias"], None)
    assert call() == _abi.ISPA_OK                          # no groups: no-op
    assert call(dt=5) == _abi.ISPA_E_UNSUPPORTED
    assert call(width=260) == _abi.ISPA_E_UNSUPPORTED      # not a multiple of 8
    assert call(width=0) == _abi.ISPA_E_ARG
    assert call(n=-1) == _abi.ISPA_E_ARG
    assert call(G=-1) == _abi.ISPA_E_ARG
    assert call(G=(1 << 26) + 1) == _abi.ISPA_E_ARG
    assert call(G=3, off=None) == _abi.ISPA_E_ARG
    assert call(G=3, off=FAKE + 2) == _abi.ISPA_E_ARG
    assert call(G=3, k=MISALIGNED) == _abi.ISPA_E_ARG
    assert call(G=3, mem=None) == _abi.ISPA_E_ARG
    assert call(G=3, in_stride=248) == _abi.ISPA_E_ARG
    assert call(G=3, in_stride=260) == _abi.ISPA_E_ARG
    assert call(G=3, ko=None) == _abi.ISPA_E_ARG
    assert call(G=3, vo=MISALIGNED) == _abi.ISPA_E_ARG
    assert call(G=3, out_stride=128) == _abi.ISPA_E_ARG
    assert call(G=3, bias=FAKE + 1) == _abi.ISPA_E_ARG


def test_fp8_argument_errors(L):
    hs, qz = L.ispa_fp8_head_scales, L.ispa_fp8_quantize
    assert hs(2, FAKE, 10, 2, 128, 256, FAKE2, None) == _abi.ISPA_E_UNSUPPORTED      # dtype
    assert hs(1, FAKE, 10, 2, 96, 256, FAKE2, None) == _abi.ISPA_E_UNSUPPORTED       # head_dim
    assert hs(1, FAKE, -1, 2, 128, 256, FAKE2, None) == _abi.ISPA_E_ARG
    assert hs(1, MISALIGNED, 10, 2, 128, 256, FAKE2, None) == _abi.ISPA_E_ARG
    assert hs(1, FAKE, 10, 2, 128, 255, FAKE2, None) == _abi.ISPA_E_ARG
    assert hs(1, FAKE, 10, 2, 128, 256, None, None) == _abi.ISPA_E_ARG
    assert qz(1, FAKE, 0, 2, 128, 256, None, None, 0, None) == _abi.ISPA_OK          # no rows: no-op
    assert qz(1, FAKE, 10, 2, 128, 256, FAKE2, FAKE + 4, 256, None) == _abi.ISPA_E_ARG   # out misaligned
    assert qz(1, FAKE, 10, 2, 128, 256, FAKE2, FAKE, 200, None) == _abi.ISPA_E_ARG   # out stride short
    at = L.ispa_attn_dual_fp8

    def call(dh=128, q=FAKE, n_q=32, qs=256, sink=None, cur=None, hist=None, a_loc=FAKE, sq=FAKE2, sk=FAKE2):
        sink = sink if sink is not None else seg()
        cur = cur if cur is not None else seg()
        hist = hist if hist is not None else seg()
        return at(2, dh, ctypes.c_float(0.088), q, n_q, qs, sq, sink, cur, hist, sk, a_loc, FAKE2, None, None,
                  None, None)
    assert call(dh=64) == _abi.ISPA_E_UNSUPPORTED
    assert call(sink=seg(n=0), cur=seg(n=0)) == _abi.ISPA_E_ARG
    assert call(hist=seg(stride=264)) == _abi.ISPA_E_ARG        # K rows need a multiple of 16
    assert call(qs=264) == _abi.ISPA_E_ARG
    assert call(sq=None) == _abi.ISPA_E_ARG
    assert call(sk=FAKE + 2) == _abi.ISPA_E_ARG
    assert call(a_loc=None) == _abi.ISPA_E_ARG
    assert call(n_q=0) == _abi.ISPA_OK


def test_balanced_argument_errors(L):
    f = L.ispa_attn_dual_balanced

    def call(dt=1, H=2, dh=128, n_q=32, sink=None, cur=None, hist=None, a_loc=FAKE, ws=None, wsb=0):
        sink = sink if sink is not None else seg()
        cur = cur if cur is not None else seg()
        hist = hist if hist is not None else seg()
        return f(dt, H, dh, ctypes.c_float(0.088), FAKE, n_q, 256, sink, cur, hist, a_loc, FAKE2, None, None, None,
                 ws, wsb, None)
    assert call(H=0) == _abi.ISPA_E_ARG
    assert call(dh=96) == _abi.ISPA_E_UNSUPPORTED
    assert call(dt=7) == _abi.ISPA_E_UNSUPPORTED
    assert call(sink=seg(n=0), cur=seg(n=0)) == _abi.ISPA_E_ARG
    assert call(a_loc=None) == _abi.ISPA_E_ARG
    assert call(n_q=0) == _abi.ISPA_OK
    assert L.ispa_attn_dual_balanced_workspace(1, 0, 128, 4680, 100, 100) == 0
    assert L.ispa_attn_dual_balanced_workspace(1, 12, 128, 4680, -1, 100) == 0
    assert L.ispa_attn_dual_balanced_workspace(0, 12, 128, 4680, 9360, 9360) == 0   # fp32: plain schedule


def test_fp8_pv_argument_errors(L):
    at = L.ispa_attn_dual_fp8_pv

    def call(dh=128, n_q=32, qs=256, sink=None, cur=None, hist=None, sq=FAKE2, sk=FAKE2, sv=FAKE2, a_loc=FAKE):
        sink = sink if sink is not None else seg()
        cur = cur if cur is not None else seg()
        hist = hist if hist is not None else seg()
        return at(2, dh, ctypes.c_float(0.088), FAKE, n_q, qs, sq, sink, cur, hist, sk, sv, a_loc, FAKE2, None,
                  None, None, None)
    assert call(sv=None) == _abi.ISPA_E_ARG                     # the value scales are required
    assert call(sv=FAKE + 2) == _abi.ISPA_E_ARG
    assert call(sv=None, n_q=0) == _abi.ISPA_E_ARG              # even when there is nothing to compute
    assert call(dh=64) == _abi.ISPA_E_UNSUPPORTED
    assert call(cur=seg(v=MISALIGNED)) == _abi.ISPA_E_ARG
    assert call(cur=seg(stride=1 << 23)) == _abi.ISPA_E_UNSUPPORTED
    assert call(sink=seg(n=0), cur=seg(n=0)) == _abi.ISPA_E_ARG
    assert call(sk=None) == _abi.ISPA_E_ARG
    assert call(n_q=0) == _abi.ISPA_OK


def test_fp8_pv_binding_checks_code_types():
    torch = pytest.importorskip("torch")
    q = torch.zeros((4, 2, 128), dtype=torch.uint8)
    s = torch.ones(2)
    k = torch.zeros((8, 2, 128), dtype=torch.uint8)
    vb = torch.zeros((8, 2, 128), dtype=torch.bfloat16)
    out = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="e4m3"):
        ispa.ispa_attn_dual_fp8_pv(q, s, None, None, k, vb, None, None, s, s, 0.088, out)
    with pytest.raises(ValueError, match="bfloat16"):
        ispa.ispa_attn_dual_fp8(q, s, None, None, k, k, None, None, s, 0.088, out)


def test_accumulate_fp8_argument_errors(L):
    f = L.ispa_absorb_accumulate_fp8

    def call(n=10, d=256, hd=128, al=FAKE, sl=FAKE2, af=FAKE, sf=FAKE2, G=FAKE, X=FAKE, F=FAKE):
        return f(n, d, hd, al, sl, af, sf, G, X, F, None, 0, None)
    assert call(hd=96) == _abi.ISPA_E_UNSUPPORTED
    assert call(d=192) == _abi.ISPA_E_UNSUPPORTED          # not a multiple of head_dim 128
    assert call(d=100, hd=64) == _abi.ISPA_E_UNSUPPORTED
    assert call(n=-1) == _abi.ISPA_E_ARG
    assert call(G=None) == _abi.ISPA_E_ARG
    assert call(al=MISALIGNED) == _abi.ISPA_E_ARG
    assert call(sf=None) == _abi.ISPA_E_ARG
    assert call(n=0, al=None, af=None, sl=None, sf=None) == _abi.ISPA_OK


def test_future_scores_argument_errors(L):
    f = L.ispa_future_scores
    base = dict(dt=1, H=2, dh=128, scale=0.088, q=FAKE, n_p=10, q_stride=256, sink=seg(n=8), cur=seg(n=8),
                hist=seg(n=16), scores=FAKE2, shs=32, lam=0.5, hist_tok=None, tok=None, ws=FAKE, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["dt"], a["H"], a["dh"], ctypes.c_float(a["scale"]), a["q"], a["n_p"], a["q_stride"], a["sink"],
                 a["cur"], a["hist"], a["scores"], a["shs"], ctypes.c_float(a["lam"]), a["hist_tok"], a["tok"],
                 a["ws"], a["ws_bytes"], None)
    assert call(dt=0) == _abi.ISPA_E_UNSUPPORTED                  # bf16 only
    assert call(dh=96) == _abi.ISPA_E_UNSUPPORTED
    assert call(H=0) == _abi.ISPA_E_ARG
    assert call(n_p=0) == _abi.ISPA_E_ARG                          # no proxies: no mean
    assert call(scale=0.0) == _abi.ISPA_E_ARG
    assert call(lam=float("inf")) == _abi.ISPA_E_ARG
    assert call(sink=seg(n=0), cur=seg(n=0), hist=seg(n=0)) == _abi.ISPA_E_ARG   # no keys
    assert call(hist=seg(k=MISALIGNED, n=16)) == _abi.ISPA_E_ARG
    assert call(cur=seg(stride=260, n=8)) == _abi.ISPA_E_ARG
    assert call(sink=seg(stride=1 << 23, n=8)) == _abi.ISPA_E_UNSUPPORTED
    assert call(q=MISALIGNED) == _abi.ISPA_E_ARG
    assert call(q_stride=128) == _abi.ISPA_E_ARG
    assert call(scores=None) == _abi.ISPA_E_ARG
    assert call(shs=31) == _abi.ISPA_E_ARG                         # head stride below the 32 keys
    assert call(tok=FAKE + 2) == _abi.ISPA_E_ARG
    assert call(ws=None) == _abi.ISPA_E_WORKSPACE
    assert call(ws_bytes=L.ispa_future_scores_workspace(2, 10) - 1) == _abi.ISPA_E_WORKSPACE
    # lse rows (fp32 [H, n_p], 256-byte rounded) + split partial states (splits x [H, n_p] float2):
    # 2 heads x 1 tile of 256 proxies -> 16 splits (capped); 12 heads x 19 tiles -> 1 split;
    # 12 heads x 7 tiles (1560 proxies) -> 3 splits
    assert L.ispa_future_scores_workspace(2, 10) == 256 + 16 * 2 * 10 * 8
    assert L.ispa_future_scores_workspace(12, 4680) == 878 * 256 + 12 * 4680 * 8
    assert L.ispa_future_scores_workspace(12, 1560) == 75008 + (3 * 12 * 1560 * 8 + 255) // 256 * 256


def test_accumulate_argument_errors(L):
    f = L.ispa_absorb_accumulate
    assert f(1, 100, 100, FAKE, FAKE2, FAKE, FAKE, FAKE, None, 0, None) == _abi.ISPA_E_UNSUPPORTED
    assert f(1, -1, 128, FAKE, FAKE2, FAKE, FAKE, FAKE, None, 0, None) == _abi.ISPA_E_ARG
    assert f(1, 10, 128, FAKE, FAKE2, None, FAKE, FAKE, None, 0, None) == _abi.ISPA_E_ARG
    assert f(1, 10, 128, MISALIGNED, FAKE2, FAKE, FAKE, FAKE, None, 0, None) == _abi.ISPA_E_ARG
    assert f(3, 10, 128, FAKE, FAKE2, FAKE, FAKE, FAKE, None, 0, None) == _abi.ISPA_E_UNSUPPORTED
    assert f(1, 0, 128, None, None, FAKE, FAKE, None, None, 0, None) == _abi.ISPA_OK
    assert L.ispa_absorb_accumulate_workspace(4680, 1536) == 0


def ptrs(n, base=FAKE):
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        arr[i] = base + 0x1000 * i
    return arr


def test_accumulate_batched_argument_errors(L):
    f = L.ispa_absorb_accumulate_batched
    b = 3
    P = ptrs(b)
    assert f(2, 100, 1536, b, P, P, P, P, P, None) == _abi.ISPA_E_UNSUPPORTED      # dtype
    assert f(1, 100, 1000, b, P, P, P, P, P, None) == _abi.ISPA_E_UNSUPPORTED      # d % 64
    assert f(1, -1, 1536, b, P, P, P, P, P, None) == _abi.ISPA_E_ARG
    assert f(1, 100, 1536, -1, P, P, P, P, P, None) == _abi.ISPA_E_ARG
    assert f(1, 100, 1536, 0, None, None, None, None, None, None) == _abi.ISPA_OK
    assert f(1, 100, 1536, b, None, P, P, P, P, None) == _abi.ISPA_E_ARG
    assert f(1, 100, 1536, b, P, P, None, P, P, None) == _abi.ISPA_E_ARG
    bad = ptrs(b)
    bad[2] = MISALIGNED
    assert f(1, 100, 1536, b, bad, P, P, P, P, None) == _abi.ISPA_E_ARG
    assert f(1, 100, 1536, b, P, P, P, bad, P, None) == _abi.ISPA_E_ARG
    assert f(1, 0, 1536, b, None, None, P, P, None, None) == _abi.ISPA_OK              # no rows: no-op


def test_solve_argument_errors_and_workspace(L):
    d, b = 256, 3
    need = L.ispa_absorb_solve_workspace(d, b)
    assert need >= 3 * d * d * 4 * b
    assert L.ispa_absorb_solve_workspace(1536, 30) == 30 * L.ispa_absorb_solve_workspace(1536, 1)
    s = L.ispa_absorb_solve
    P = ptrs(b)
    assert s(100, b, ctypes.c_float(1e-2), P, P, P, 0, P, FAKE, FAKE, need, None) == _abi.ISPA_E_UNSUPPORTED
    assert s(d, b, ctypes.c_float(-1.0), P, P, P, 0, P, FAKE, FAKE, need, None) == _abi.ISPA_E_ARG
    assert s(d, b, ctypes.c_float(1e-2), P, P, P, 0, P, FAKE, FAKE, need - 1, None) == _abi.ISPA_E_WORKSPACE
    assert s(d, b, ctypes.c_float(1e-2), P, P, P, 0, P, None, FAKE, need, None) == _abi.ISPA_E_ARG
    bad = ptrs(b)
    bad[1] = MISALIGNED
    assert s(d, b, ctypes.c_float(1e-2), P, bad, P, 0, P, FAKE, FAKE, need, None) == _abi.ISPA_E_ARG
    assert s(d, 0, ctypes.c_float(1e-2), None, None, None, 0, None, None, None, 0, None) == _abi.ISPA_OK


def test_solve_eps_argument_errors_and_workspace(L):
    d, b = 256, 3
    need = L.ispa_absorb_solve_eps_workspace(d, b)
    # the solve's workspace plus 4 terms x 3 layers x 32 tile partials (4 tiles, rounded up to 32 doubles)
    assert need == L.ispa_absorb_solve_workspace(d, b) + 4 * b * 32 * 8
    s = L.ispa_absorb_solve_eps
    P = ptrs(b)
    ok = lambda **kw: dict(dict(d=d, lam=1e-2, F=P, info=FAKE, eps=FAKE2, ref=None, ws=FAKE, nbytes=need), **kw)
    call = lambda a: s(a["d"], b, ctypes.c_float(a["lam"]), P, P, a["F"], P, 0, P, a["info"], a["eps"], a["ref"],
                       a["ws"], a["nbytes"], None)
    assert call(ok(d=100)) == _abi.ISPA_E_UNSUPPORTED
    assert call(ok(lam=-1.0)) == _abi.ISPA_E_ARG
    assert call(ok(nbytes=need - 1)) == _abi.ISPA_E_WORKSPACE
    assert call(ok(ws=None)) == _abi.ISPA_E_WORKSPACE
    assert call(ok(ws=FAKE + 16)) == _abi.ISPA_E_ARG          # 256-byte alignment
    assert call(ok(info=None)) == _abi.ISPA_E_ARG
    assert call(ok(eps=None)) == _abi.ISPA_E_ARG
    assert call(ok(eps=FAKE2 + 4)) == _abi.ISPA_E_ARG
    assert call(ok(ref=FAKE + 4)) == _abi.ISPA_E_ARG
    assert call(ok(F=None)) == _abi.ISPA_E_ARG
    bad = ptrs(b)
    bad[2] = MISALIGNED
    assert call(ok(F=bad)) == _abi.ISPA_E_ARG
    assert s(d, 0, ctypes.c_float(1e-2), None, None, None, None, 0, None, None, None, None, None, 0, None) == \
        _abi.ISPA_OK


def test_error_argument_errors_and_workspace(L):
    d, b = 128, 2
    need = L.ispa_layer_error_workspace(d, b)
    assert need >= 2 * d * d * 4 * b
    f = L.ispa_layer_error
    P = ptrs(b)
    assert f(d, b, P, P, P, P, 0, P, FAKE, None, FAKE, need - 8, None) == _abi.ISPA_E_WORKSPACE
    assert f(d, b, P, P, P, P, 0, P, None, None, FAKE, need, None) == _abi.ISPA_E_ARG
    assert f(96, b, P, P, P, P, 0, P, FAKE, None, FAKE, need, None) == _abi.ISPA_E_UNSUPPORTED


def test_rank_layers_matches_oracle():
    rng = np.random.default_rng(0)
    for trial in range(50):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(0, n + 1))
        eps = rng.integers(0, 6, size=n).astype(float) * rng.choice([1.0, 1e-3])
        if trial % 7 == 0:
            eps[rng.integers(0, n)] = np.nan
        sel, flags = ispa.ispa_rank_layers(eps.tolist(), k)
        ref_sel, ref_mask = oab.rank_layers(eps, k)
        assert sel == ref_sel.tolist()
        assert flags == ref_mask.astype(int).tolist()


def test_rank_layers_errors(L):
    e = (ctypes.c_double * 3)(1.0, 2.0, 3.0)
    sel = (ctypes.c_int32 * 4)()
    assert L.ispa_rank_layers(e, 3, 4, sel, None) == _abi.ISPA_E_ARG
    assert L.ispa_rank_layers(e, 3, -1, sel, None) == _abi.ISPA_E_ARG
    assert L.ispa_rank_layers(None, 3, 1, sel, None) == _abi.ISPA_E_ARG
    assert L.ispa_rank_layers(e, 3, 0, None, None) == _abi.ISPA_OK


def test_steady_state_argument_errors(L):
    ok, arg, uns = _abi.ISPA_OK, _abi.ISPA_E_ARG, _abi.ISPA_E_UNSUPPORTED
    # weight update
    assert L.ispa_apply_delta(0, 8, FAKE, FAKE2, 0, FAKE, None) == arg
    assert L.ispa_apply_delta(8, 8, None, FAKE2, 0, FAKE, None) == arg
    assert L.ispa_apply_delta(8, 8, FAKE, FAKE2, 0, None, None) == arg
    assert L.ispa_apply_delta(8, 8, MISALIGNED, FAKE2, 0, FAKE, None) == arg
    # projection
    assert L.ispa_project(0, 64, 64, None, 64, None, None, 64, None) == ok      # empty: no-op
    assert L.ispa_project(-1, 64, 64, FAKE, 64, FAKE2, FAKE, 64, None) == arg
    assert L.ispa_project(10, 48, 64, FAKE, 48, FAKE2, FAKE, 64, None) == uns  # d_in % 32
    assert L.ispa_project(10, 64, 60, FAKE, 64, FAKE2, FAKE, 64, None) == uns  # d_out % 8
    assert L.ispa_project(10, 64, 64, FAKE, 60, FAKE2, FAKE, 64, None) == arg  # lda < d_in
    assert L.ispa_project(10, 64, 64, FAKE, 68, FAKE2, FAKE, 64, None) == arg  # lda % 8
    assert L.ispa_project(10, 64, 64, FAKE, 64, FAKE2, FAKE, 56, None) == arg  # ldy < d_out
    assert L.ispa_project(10, 64, 64, MISALIGNED, 64, FAKE2, FAKE, 64, None) == arg
    assert L.ispa_project(10, 64, 64, FAKE, 64, None, FAKE, 64, None) == arg
    # eviction plan (host only)
    kept = (ctypes.c_int64 * 3)()
    assert L.ispa_kv_plan(3, None, 1, 2, 3, kept, None) == arg
    flags = (ctypes.c_uint8 * 3)(1, 0, 1)
    assert L.ispa_kv_plan(3, flags, 1, -2, 3, kept, None) == arg
    assert L.ispa_kv_plan(0, None, 1, 2, 3, None, None) == ok


def test_kv_plan_matches_oracle():
    from oracle import steady as ost
    rng = np.random.default_rng(4)
    for _ in range(20):
        n = int(rng.integers(0, 40))
        flags = rng.integers(0, 2, size=n).tolist()
        ns, nh, nc = (int(x) for x in rng.integers(0, 100000, size=3))
        kept, ev = ispa.ispa_kv_plan(flags, ns, nh, nc)
        ref = ost.layer_plan([bool(f) for f in flags], ns, nh, nc)
        assert kept == ref["hist_kept"]
        assert ev == ref["evicted_tokens"]


def test_absorb_bindings_validate_every_entry():
    """The Python binding checks every per-layer matrix and output vector before the library is called
    (a wrong dtype or a short vector would otherwise let the kernels write out of bounds)."""
    import torch
    import kv_cache_attention_split_amd as ispa
    d = 64
    m = lambda dt=torch.float32, shape=(d, d): torch.zeros(shape, dtype=dt)
    ws = torch.zeros(16, dtype=torch.uint8)
    info = torch.zeros(2, dtype=torch.int32)
    eps = torch.zeros(2, dtype=torch.float64)
    good = [m(), m()]
    cases = [
        lambda: ispa.ispa_absorb_solve([m(), m(torch.float64)], good, good, good, 1e-2, info, ws),
        lambda: ispa.ispa_absorb_solve(good, [m(), m(shape=(d, d + 8))], good, good, 1e-2, info, ws),
        lambda: ispa.ispa_absorb_solve(good, good, [m(), m().t()], good, 1e-2, info, ws),
        lambda: ispa.ispa_absorb_solve(good, good, good, [m()], 1e-2, info, ws),
        lambda: ispa.ispa_absorb_solve(good, good, good, good, 1e-2, info.to(torch.int64), ws),
        lambda: ispa.ispa_absorb_solve(good, good, good, good, 1e-2, info[:1], ws),
        lambda: ispa.ispa_absorb_solve(good, good, good, good, 1e-2, None, ws),
        lambda: ispa.ispa_layer_error(good, good, good, good, good, eps.to(torch.float32), None, ws),
        lambda: ispa.ispa_layer_error(good, good, good, good, good, eps[:1], None, ws),
        lambda: ispa.ispa_layer_error(good, good, good, good, good, eps, eps[:1], ws),
        lambda: ispa.ispa_layer_error(good, good, [m(), m(torch.bfloat16)], good, good, eps, None, ws),
        lambda: ispa.ispa_absorb_accumulate(m(torch.bfloat16, (10, d)), m(torch.bfloat16, (10, d)), m(), m(torch.float64)),
        lambda: ispa.ispa_absorb_accumulate(m(torch.bfloat16, (10, d)), m(torch.bfloat16, (10, d)), m(), m(), m(shape=(d, 8))),
        lambda: ispa.ispa_absorb_accumulate_fp8(m(torch.uint8, (10, d)), m(shape=(1,)), m(torch.uint8, (10, d)),
                                                m(shape=(1,)), 64, m(), m(torch.float64)),
        lambda: ispa.ispa_absorb_accumulate_fp8(m(torch.uint8, (10, d)), m(shape=(1,)), m(torch.uint8, (10, d)),
                                                m(torch.float64, (1,)), 64, m(), m()),
    ]
    for i, call in enumerate(cases):
        with pytest.raises(ValueError):
            call()
    # well-formed arguments that live in host memory are refused too (the library takes device pointers)
    with pytest.raises(ValueError, match="GPU tensor"):
        ispa.ispa_absorb_solve(good, good, good, good, 1e-2, info, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        ispa.ispa_layer_error(good, good, good, good, good, eps, None, ws)
