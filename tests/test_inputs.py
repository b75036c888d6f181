"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

import ispa_inputs as inputs


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact ties between two bf16 values, both parities
                        ((np.arange(1000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)[1:]])
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_segment_sizes():
    c2 = inputs.CONFIGS[2].segment_sizes(0)
    assert c2 == {"n_q": 4680, "n_sink": 4680, "n_cur": 4680, "n_hist": 9360}
    c5 = inputs.CONFIGS[5].segment_sizes(0)
    assert c5 == {"n_q": 4680, "n_sink": 4680, "n_cur": 4680, "n_hist": 93600}
    c3 = [inputs.CONFIGS[3].segment_sizes(c) for c in range(4)]
    assert [c["n_sink"] for c in c3] == [0, 4680, 4680, 4680]
    assert [c["n_hist"] for c in c3] == [0, 0, 4680, 9360]
    assert inputs.CONFIGS[4].d == 5120 and inputs.CONFIGS[3].d == 1536
    assert inputs.CONFIGS[1].segment_sizes() == {"n_q": 128, "n_sink": 64, "n_cur": 128, "n_hist": 512}


def test_seeding_is_deterministic_and_distinct():
    a = inputs.attention_inputs(1)
    b = inputs.attention_inputs(1)
    for k in ("q", "cur_k", "hist_v"):
        np.testing.assert_array_equal(a[k], b[k])
    w0, w1 = inputs.weight(1, 0), inputs.weight(1, 1)
    assert not np.array_equal(w0, w1)
    assert abs(w0.std() * np.sqrt(128) - 1.0) < 0.05


def test_absorb_rows_shapes_and_empty_history_chunks():
    r0 = inputs.absorb_rows(3, 0, 0, n_rows=64)
    assert r0["a_loc"].shape == (64, 1536)
    np.testing.assert_array_equal(r0["a_loc"], r0["a_full"])      # chunk 0 has no history
    r3 = inputs.absorb_rows(3, 0, 3, n_rows=64)
    assert not np.array_equal(r3["a_loc"], r3["a_full"])
    # bf16 values
    np.testing.assert_array_equal(inputs.round_bf16(r3["a_full"]), r3["a_full"])
