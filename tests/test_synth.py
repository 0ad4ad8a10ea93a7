"""The seeded input generator: determinism, rounding and distributions (CPU)."""
import numpy as np
import torch

import synth


def test_same_seed_same_bits_and_different_seed_differs():
    a = synth.make_norm_gemm("t", 8, 32, 16, seed=3)
    b = synth.make_norm_gemm("t", 8, 32, 16, seed=3)
    c = synth.make_norm_gemm("t", 8, 32, 16, seed=4)
    for k in ("x", "gamma", "beta", "W", "bias"):
        assert np.array_equal(a.arrays[k], b.arrays[k])
    assert not np.array_equal(a.arrays["x"], c.arrays["x"])


def test_chunked_draw_equals_one_shot_draw(monkeypatch):
    rng1 = np.random.Generator(np.random.PCG64(5))
    one = synth.normal_bits(rng1, (1000,), 0.0, 1.0, synth.F16)
    monkeypatch.setattr(synth, "_CHUNK", 77)
    rng2 = np.random.Generator(np.random.PCG64(5))
    many = synth.normal_bits(rng2, (1000,), 0.0, 1.0, synth.F16)
    assert np.array_equal(one, many)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 10, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, 3.0e38, -1.5, 65504.0], np.float32)])
    ours = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_rounding_is_numpy_rne():
    v = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65520.0], dtype=np.float32)
    bits = synth.f32_to_f16_bits(v)
    # ties go to even: 1+2^-11 -> 1.0, 1+3*2^-11 -> 1+2^-9... (even mantissa), 65520 -> inf
    assert bits[0] == 0x3C00 and bits[1] == 0x3C02 and bits[2] == 0x7C00


def test_distributions_follow_mean_and_variance_reading():
    case = synth.make_norm_gemm("t", 64, 4096, 64, seed=1)
    x = case.arrays["x"].view(np.float16).astype(np.float64)
    g = case.arrays["gamma"].view(np.float16).astype(np.float64)
    W = case.arrays["W"].view(np.float16).astype(np.float64)
    assert abs(x.mean()) < 0.02 and abs(x.var() - 1.0) < 0.02
    assert abs(g.mean() - 1.0) < 0.02 and abs(g.var() - 0.1) < 0.01
    assert abs(W.var() * 4096 - 1.0) < 0.05


def test_workload_shapes():
    c = synth.ln_linear_bias_64x256()
    assert c.arrays["x"].shape == (64, 256) and c.arrays["W"].shape == (256, 256)
    assert c.arrays["bias"].shape == (256,) and c.norm == synth.NORM_LAYERNORM
    d = synth.make_ffn("f", 4, 16, 24, 8)
    assert d.arrays["W1"].shape == (24, 16) and d.arrays["W2"].shape == (8, 24)
