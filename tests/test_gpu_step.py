"""The whole warmup step at the 1.3B model's scale, run twice: the same bits every time.

30 layers x 4 chunks of dual-stream attention (12 heads x 128, 4680 queries, history growing 0 -> 6
frames), the statistics of every chunk, one batched solve and one batched error over the 30 layers, and
the ranking. Every kernel on this path reduces in a fixed order, so two runs must agree bit for bit in
A_loc / A_full, G / X / F, dW and eps, and select the same layers. Launches this large hold more
workgroups than the CUs run at once, which is where a workgroup that reads what another one has already
overwritten shows (the per-stage parity tests against the oracle use smaller batches). Inputs are drawn
on the device (bf16 N(0, 1) keys, values and queries, W ~ N(0, 1/d)): this test is about repeatability;
the oracle comparisons of each stage live in the other test files.
"""
import numpy as np
import pytest

import ispa_inputs as inputs

from gpu_helpers import torch_mod

pytestmark = pytest.mark.gpu


def test_warmup_step_bitwise_repeatable():
    import kv_cache_attention_split_amd as ispa
    torch = torch_mod()
    wl = inputs.CONFIGS[3]
    L, H, dh, d = wl.n_layers, wl.n_heads, wl.head_dim, wl.d
    n_q, ft = inputs.CHUNK_TOKENS, inputs.FRAME_TOKENS
    print(f"case: warmup step, {L} layers x {len(wl.chunks)} chunks, {H} x {dh}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(2024)
    n_frames = max(max(c.sink[1], c.cur[1], c.hist[1]) for c in wl.chunks)

    def randn(*shape, scale=1.0):
        return (scale * torch.randn(shape, device="cuda", generator=g)).to(torch.bfloat16)

    kv = [(randn(n_frames * ft, H, dh), randn(n_frames * ft, H, dh)) for _ in range(L)]
    qs = [[randn(n_q, H, dh) for _ in wl.chunks] for _ in range(L)]
    Ws = [torch.randn((d, d), device="cuda", generator=g) / float(np.sqrt(d)) for _ in range(L)]

    def seg(li, r):
        k, v = kv[li]
        return k[r[0] * ft:r[1] * ft], v[r[0] * ft:r[1] * ft]

    def step():
        a_loc = torch.empty((n_q, d), dtype=torch.bfloat16, device="cuda")
        a_full = torch.empty_like(a_loc)
        lse = [torch.empty((H, n_q), dtype=torch.float32, device="cuda") for _ in range(3)]
        stats = [[torch.zeros((d, d), dtype=torch.float32, device="cuda") for _ in range(3)] for _ in range(L)]
        outs = []
        for li in range(L):
            for c, ch in enumerate(wl.chunks):
                ispa.ispa_attn_dual(qs[li][c], *seg(li, ch.sink), *seg(li, ch.cur), *seg(li, ch.hist), wl.scale,
                                    a_loc, a_full, lse[0], lse[1], lse[2])
                if li in (0, L - 1):
                    outs.append((a_loc.clone(), a_full.clone(), [t.clone() for t in lse]))
                ispa.ispa_absorb_accumulate(a_loc, a_full, *stats[li])
        Gs, Xs, Fs = ([s[i] for s in stats] for i in range(3))
        dW = [torch.empty((d, d), dtype=torch.float32, device="cuda") for _ in range(L)]
        info = torch.full((L,), -1, dtype=torch.int32, device="cuda")
        eps = torch.zeros((L,), dtype=torch.float64, device="cuda")
        ref = torch.zeros_like(eps)
        ws1 = torch.empty(ispa.ispa_absorb_solve_workspace(d, L), dtype=torch.uint8, device="cuda")
        ws2 = torch.empty(ispa.ispa_layer_error_workspace(d, L), dtype=torch.uint8, device="cuda")
        ispa.ispa_absorb_solve(Gs, Xs, Ws, dW, wl.lam, info, ws1)
        ispa.ispa_layer_error(Gs, Xs, Fs, Ws, dW, eps, ref, ws2)
        e = eps.cpu().numpy()
        sel, _ = ispa.ispa_rank_layers(e.tolist(), wl.k_select)
        return outs, stats, dW, info.cpu().numpy(), e, ref.cpu().numpy(), sel

    o1, s1, w1, i1, e1, r1, sel1 = step()
    o2, s2, w2, i2, e2, r2, sel2 = step()
    assert i1.tolist() == [0] * L and i2.tolist() == [0] * L
    assert np.all(np.isfinite(e1)) and np.all(e1 >= 0) and np.all(r1 > 0)
    for (a1, f1, l1), (a2, f2, l2) in zip(o1, o2):
        assert torch.equal(a1, a2) and torch.equal(f1, f2) and all(torch.equal(x, y) for x, y in zip(l1, l2))
    bad = [li for li in range(L) if not all(torch.equal(x, y) for x, y in zip(s1[li], s2[li]))]
    assert not bad, f"statistics differ in layers {bad}"
    bad = [li for li in range(L) if not torch.equal(w1[li], w2[li])]
    assert not bad, f"dW differs in layers {bad}"
    assert np.array_equal(e1, e2) and np.array_equal(r1, r2)
    assert sel1 == sel2
    print(f"   eps / ref in [{float(np.min(e1 / r1)):.3f}, {float(np.max(e1 / r1)):.3f}], selected {sel1}",
          flush=True)
