"""The seeded input generator: deterministic draws and correct dtype rounding."""

import numpy as np
import torch

from synth import CONFIGS, bf16_bits_to_f64, draw, f64_to_bf16_bits


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-20, 20, 100000))).astype(np.float32)
    # include exact ties (low 16 bits == 0x8000) both with even and odd kept bits
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_draws_are_deterministic_and_ordered():
    a = draw(5, [((2, 3), 1.0), ((4,), 0.5)], "bf16")
    b = draw(5, [((2, 3), 1.0), ((4,), 0.5)], "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x.bits, y.bits)
    c = draw(5, [((2, 3), 1.0)], "f32")
    rng = np.random.default_rng(5)
    assert np.array_equal(c[0].bits, (rng.standard_normal((2, 3)) * 1.0).astype(np.float32))


def test_workload_shapes():
    w = CONFIGS["retention_7b_8k"]
    q, k, v, g = w.inputs(batch=1, seqlen=8)
    assert q.bits.shape == (1, 8, 16, 256) and q.bits.dtype == np.uint16
    assert g is not None and g.f64.shape == (1, 8, 16, 256)
    t = CONFIGS["tiny_fp32"]
    q, k, v, g = t.inputs()
    assert g is None and q.bits.dtype == np.float32 and q.bits.shape == (1, 256, 2, 64)
    assert q.torch().dtype == torch.float32
