"""The seeded generators: bf16 rounding, layout and determinism."""

import numpy as np
import torch

from head_latent_attention_16_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-40, -3.0e38, np.inf, -np.inf], np.float32)])
    ours = I.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(I.bf16_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_workloads_deterministic_and_laid_out():
    a = I.uniform(B=2, T=8)
    b = I.uniform(B=2, T=8)
    assert np.array_equal(a.cache, b.cache) and np.array_equal(a.q_C, b.q_C)
    assert a.cache.shape == (16, 576) and a.cache.dtype == np.uint16
    assert list(a.offsets) == [0, 8, 16]
    r = I.ragged(B=5, lo=3, hi=9)
    assert np.array_equal(r.lens, I.ragged_lens(B=5, lo=3, hi=9))
    assert np.all((r.lens >= 3) & (r.lens <= 9))
    assert r.offsets[-1] == r.lens.sum()
    L = I.layer(B=3, lo=4, hi=6)
    assert np.all(np.diff(L.offsets) == L.lens + 1)      # one free row per sequence
    assert L.W["W_UQ"].shape == (128 * 192, 1536) and L.W["W_O"].shape == (7168, 16384)
    t = I.tiny()
    assert t.dtype == "f32" and t.kv_raw.shape == (1, 64, 40) and t.q_C.shape == (1, 4, 16)
    c = I.causal(B=3, T=10, n_q=4)
    assert c.n_q == 4 and c.q_C.shape == (12, 128, 128) and c.q_R.shape == (12, 128, 64)
    assert c.cache.shape == (30, 576) and list(c.lens) == [10, 10, 10]


def test_weight_std_is_fan_in_inverse_sqrt():
    L = I.layer(B=2, lo=4, hi=4)
    for name, fan_in in (("W_DQ", 7168), ("W_UQ", 1536), ("W_UK", 512), ("W_O", 16384)):
        s = float(np.std(I.bf16_to_f32(L.W[name]).astype(np.float64)))
        assert abs(s * np.sqrt(fan_in) - 1.0) < 0.01, name
