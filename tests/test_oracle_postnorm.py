"""Pins of the oracle's post-GEMM normalization (CPU only): against the
unfused torch composition in fp64 (linear, then layer_norm / rms_norm over
the output row), the normalization invariants, the identity weight (which
turns it into the prologue normalization of x) and a hand-worked row."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth

LN, RMS = synth.NORM_LAYERNORM, synth.NORM_RMSNORM


def val(bits, dtype=synth.F16):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == synth.F16:
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def draw(M, N, K, dtype, seed, bias=True, gamma=True, beta=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = synth.normal_bits(rng, (M, K), 0.0, 1.0, dtype)
    W = synth.normal_bits(rng, (N, K), 0.0, 1.0 / K, dtype)
    b = synth.normal_bits(rng, (N,), 0.0, 0.1, dtype) if bias else None
    g = synth.normal_bits(rng, (N,), 1.0, 0.1, dtype) if gamma else None
    be = synth.normal_bits(rng, (N,), 0.0, 0.1, dtype) if beta else None
    return x, W, b, g, be


@pytest.mark.parametrize("norm", [LN, RMS])
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("bias,gamma,beta", [(True, True, True), (False, True, False),
                                             (True, False, False)])
def test_matches_torch_linear_then_norm(norm, dtype, bias, gamma, beta):
    x, W, b, g, be = draw(5, 37, 23, dtype, 11, bias, gamma, beta)
    got = oracle.gemm_norm(x, W, b, g, be, 0.5, norm, dtype)
    t = lambda a: None if a is None else torch.from_numpy(val(a, dtype))
    z = Fn.linear(t(x), t(W), t(b))
    if norm == LN:
        ref = Fn.layer_norm(z, (37,), t(g), t(be), eps=float(np.float32(0.5)))
    else:
        ref = Fn.rms_norm(z, (37,), t(g), eps=float(np.float32(0.5)))
        if be is not None:
            ref = ref + t(be)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rms_invariant_and_layernorm_mean_zero():
    x, W, b, _, _ = draw(6, 64, 48, synth.F16, 3, gamma=False, beta=False)
    y = oracle.gemm_norm(x, W, b, None, None, 1e-5, RMS, synth.F16)
    z = val(x) @ val(W).T + val(b)
    ms = (z * z).mean(axis=1)
    assert np.allclose((y * y).mean(axis=1), ms / (ms + np.float64(np.float32(1e-5))), atol=1e-12)
    yl = oracle.gemm_norm(x, W, b, None, None, 1e-5, LN, synth.F16)
    assert np.allclose(yl.mean(axis=1), 0.0, atol=1e-12)


def test_identity_weight_normalizes_x_itself():
    """W = I, no bias: z = x, so the post-GEMM norm is the prologue norm of x."""
    x, _, _, g, be = draw(4, 32, 32, synth.F16, 5)
    eye = synth.f32_to_f16_bits(np.eye(32, dtype=np.float32))
    for norm in (LN, RMS):
        got = oracle.gemm_norm(x, eye, None, g, be, 1e-5, norm, synth.F16)
        assert np.allclose(got, oracle.normalize(x, g, be, 1e-5, norm, synth.F16), atol=1e-12)


def test_hand_worked_row():
    # x = [1, 2], W = [[1, 0], [0, 1], [1, 1], [1, -1]]: z = [1, 2, 3, -1]
    # RMSNorm: mean z^2 = 15 / 4, y = z / sqrt(3.75) (eps 0);  LayerNorm: mu = 1.25,
    # var = (0.0625 + 0.5625 + 3.0625 + 5.0625) / 4 = 2.1875
    f = lambda v: synth.f32_to_f16_bits(np.array(v, dtype=np.float32))
    x, W = f([[1, 2]]), f([[1, 0], [0, 1], [1, 1], [1, -1]])
    z = np.array([1.0, 2.0, 3.0, -1.0])
    assert np.allclose(oracle.gemm_norm(x, W, None, None, None, 0.0, RMS, synth.F16)[0],
                       z / np.sqrt(3.75), atol=1e-15)
    assert np.allclose(oracle.gemm_norm(x, W, None, None, None, 0.0, LN, synth.F16)[0],
                       (z - 1.25) / np.sqrt(2.1875), atol=1e-15)


def test_column_sampling_and_errors():
    x, W, b, g, be = draw(3, 20, 8, synth.F16, 2)
    full = oracle.gemm_norm(x, W, b, g, be, 1e-5, LN, synth.F16)
    part = oracle.gemm_norm(x, W, b, g, be, 1e-5, LN, synth.F16, rows=[2, 0], cols=[19, 3])
    assert np.array_equal(part, full[np.ix_([2, 0], [19, 3])])
    with pytest.raises(ValueError):
        oracle.gemm_norm(x, W, b, g, be, 1e-5, synth.NORM_NONE, synth.F16)
