"""Pins of the fp64 CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against a closed form, an invariant, a library
routine evaluating the pages' unfused composition, or a hand-worked example,
so that a plausible slip in the oracle (a dropped term, a wrong sign or index,
a transposed operand, eps outside the root, an unbiased variance, bias after
the activation) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(a):
    return synth.f32_to_f16_bits(np.asarray(a, dtype=np.float32))


def bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def val16(bits, dtype):
    """Decode bits with a library routine (numpy / torch), not the oracle."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == synth.F16:
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------- decoders
def test_f16_decoder_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_matches_torch_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode(bits, oracle.BF16)
    ref = val16(bits, synth.BF16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------- normalization invariants
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("K", [1, 2, 7, 256, 1000])
def test_layernorm_pre_affine_mean_zero_and_variance_ratio(dtype, K):
    rng = np.random.default_rng(K)
    x = synth.bits_from_f32(rng.normal(0.3, 2.0, size=(5, K)).astype(np.float32), dtype)
    eps = 1e-3
    a = oracle.normalize(x, None, None, eps, oracle.NORM_LAYERNORM, dtype)
    xv = val16(x, dtype)
    var = xv.var(axis=1)                       # biased, numpy
    e = float(np.float32(eps))
    assert np.all(np.abs(a.mean(axis=1)) <= 1e-12)
    np.testing.assert_allclose(a.var(axis=1), var / (var + e), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("K", [1, 3, 256, 4097])
def test_rmsnorm_pre_affine_mean_square_ratio(K):
    rng = np.random.default_rng(K + 1)
    x = f16(rng.normal(0.5, 1.5, size=(4, K)))
    eps = 1e-2
    a = oracle.normalize(x, None, None, eps, oracle.NORM_RMSNORM, synth.F16)
    ms = (val16(x, synth.F16) ** 2).mean(axis=1)
    e = float(np.float32(eps))
    np.testing.assert_allclose((a ** 2).mean(axis=1), ms / (ms + e), rtol=1e-12)
    # no mean subtraction: the sign pattern of x survives
    assert np.array_equal(np.sign(a), np.sign(val16(x, synth.F16)))


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_layernorm_with_affine_matches_torch_layer_norm(dtype):
    rng = np.random.default_rng(7)
    M, K = 6, 37
    x = synth.bits_from_f32(rng.normal(1.0, 3.0, (M, K)).astype(np.float32), dtype)
    g = synth.bits_from_f32(rng.normal(1.0, 0.3, K).astype(np.float32), dtype)
    b = synth.bits_from_f32(rng.normal(0.0, 0.3, K).astype(np.float32), dtype)
    eps = 0.5  # large, so that eps inside vs outside the root differ visibly
    a = oracle.normalize(x, g, b, eps, oracle.NORM_LAYERNORM, dtype)
    ref = Fn.layer_norm(t64(val16(x, dtype)), (K,), t64(val16(g, dtype)),
                        t64(val16(b, dtype)), eps=float(np.float32(eps))).numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-12)


def test_rmsnorm_with_gamma_matches_torch_rms_norm():
    rng = np.random.default_rng(8)
    M, K = 5, 29
    x = f16(rng.normal(0.7, 2.0, (M, K)))
    g = f16(rng.normal(1.0, 0.3, K))
    eps = 0.5
    a = oracle.normalize(x, g, None, eps, oracle.NORM_RMSNORM, synth.F16)
    ref = Fn.rms_norm(t64(val16(x, synth.F16)), (K,), t64(val16(g, synth.F16)),
                      eps=float(np.float32(eps))).numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-12)


def test_norm_none_is_identity_on_x():
    x = f16(np.linspace(-3, 3, 40).reshape(4, 10))
    a = oracle.normalize(x, f16(np.full(10, 2.0)), f16(np.ones(10)), 1e-5,
                         oracle.NORM_NONE, synth.F16)
    assert np.array_equal(a, val16(x, synth.F16))


# ------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 11), (16, 3, 9), (13, 17, 65)])
def test_gemm_without_norm_matches_numpy_matmul(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = f16(rng.normal(0, 1, (M, K)))
    W = f16(rng.normal(0, 1, (N, K)))
    bias = f16(rng.normal(0, 1, N))
    y = oracle.norm_gemm(x, None, None, W, bias, 1e-5, oracle.NORM_NONE,
                         oracle.ACT_NONE, synth.F16)
    ref = val16(x, synth.F16) @ val16(W, synth.F16).T + val16(bias, synth.F16)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


TORCH_ACT = {oracle.ACT_NONE: lambda z: z, oracle.ACT_SILU: Fn.silu, oracle.ACT_RELU: Fn.relu,
             oracle.ACT_GELU: lambda z: Fn.gelu(z, approximate="none")}


@pytest.mark.parametrize("norm,act", [(oracle.NORM_LAYERNORM, oracle.ACT_NONE),
                                      (oracle.NORM_LAYERNORM, oracle.ACT_SILU),
                                      (oracle.NORM_RMSNORM, oracle.ACT_SILU),
                                      (oracle.NORM_LAYERNORM, oracle.ACT_RELU),
                                      (oracle.NORM_RMSNORM, oracle.ACT_GELU)])
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_full_path_matches_unfused_torch_composition(norm, act, dtype):
    """The pages' op-by-op composition written with library routines in fp64."""
    rng = np.random.default_rng(11)
    M, N, K = 9, 14, 33
    enc = lambda a: synth.bits_from_f32(np.asarray(a, np.float32), dtype)
    x, g, b = enc(rng.normal(0, 1, (M, K))), enc(rng.normal(1, .3, K)), enc(rng.normal(0, .3, K))
    W, bias = enc(rng.normal(0, .2, (N, K))), enc(rng.normal(0, .3, N))
    eps = 1e-2
    y = oracle.norm_gemm(x, g, b, W, bias, eps, norm, act, dtype)
    X, G, B, Wt, Bi = (t64(val16(v, dtype)) for v in (x, g, b, W, bias))
    e = float(np.float32(eps))
    A = Fn.layer_norm(X, (K,), G, B, e) if norm == oracle.NORM_LAYERNORM \
        else Fn.rms_norm(X, (K,), G, e) + B
    Z = Fn.linear(A, Wt, Bi)
    ref = TORCH_ACT[act](Z).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_row_and_column_sampling_selects_the_right_entries():
    rng = np.random.default_rng(12)
    M, N, K = 11, 13, 20
    x, W = f16(rng.normal(0, 1, (M, K))), f16(rng.normal(0, 1, (N, K)))
    g, b, bias = f16(rng.normal(1, .3, K)), f16(rng.normal(0, .3, K)), f16(rng.normal(0, 1, N))
    full = oracle.norm_gemm(x, g, b, W, bias, 1e-5, oracle.NORM_LAYERNORM,
                            oracle.ACT_SILU, synth.F16)
    rows, cols = [10, 0, 3], [12, 5, 0, 7]
    part = oracle.norm_gemm(x, g, b, W, bias, 1e-5, oracle.NORM_LAYERNORM,
                            oracle.ACT_SILU, synth.F16, rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])


def test_identity_weight_returns_the_normalized_rows():
    rng = np.random.default_rng(13)
    K = 24
    x, g, b = f16(rng.normal(0, 1, (7, K))), f16(rng.normal(1, .3, K)), f16(rng.normal(0, .3, K))
    W = f16(np.eye(K))
    y = oracle.norm_gemm(x, g, b, W, None, 1e-5, oracle.NORM_LAYERNORM,
                         oracle.ACT_NONE, synth.F16)
    ref = Fn.layer_norm(t64(val16(x, synth.F16)), (K,), t64(val16(g, synth.F16)),
                        t64(val16(b, synth.F16)), float(np.float32(1e-5))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_SILU])
def test_constant_row_gives_act_of_beta_times_W_plus_bias(act):
    rng = np.random.default_rng(14)
    M, N, K = 3, 10, 64
    x = f16(np.full((M, K), 1.75) * np.array([[1.0], [-2.0], [0.5]]))
    g, b = f16(rng.normal(1, .3, K)), f16(rng.normal(0, .3, K))
    W, bias = f16(rng.normal(0, .3, (N, K))), f16(rng.normal(0, .3, N))
    y = oracle.norm_gemm(x, g, b, W, bias, 1e-5, oracle.NORM_LAYERNORM, act, synth.F16)
    z = val16(W, synth.F16) @ val16(b, synth.F16) + val16(bias, synth.F16)
    ref = z / (1 + np.exp(-z)) if act == oracle.ACT_SILU else z
    for m in range(M):
        np.testing.assert_allclose(y[m], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------- SiLU
def test_silu_closed_forms_via_zero_weight_and_bias_sweep():
    N, K = 41, 8
    bias_vals = np.linspace(-20, 20, N)
    bias = f16(bias_vals)
    x = f16(np.random.default_rng(15).normal(0, 1, (2, K)))
    W = f16(np.zeros((N, K)))
    y = oracle.norm_gemm(x, None, None, W, bias, 1e-5, oracle.NORM_LAYERNORM,
                         oracle.ACT_SILU, synth.F16)
    zb = val16(bias, synth.F16)
    ref = Fn.silu(t64(zb)).numpy()
    for m in range(2):
        np.testing.assert_allclose(y[m], ref, rtol=1e-14, atol=0)
    # SiLU(0) = 0 exactly (zero bias, zero weight)
    y0 = oracle.norm_gemm(x, None, None, W, None, 1e-5, oracle.NORM_LAYERNORM,
                          oracle.ACT_SILU, synth.F16)
    assert np.all(y0 == 0.0)
    # SiLU(-z) = SiLU(z) - z
    yneg = oracle.norm_gemm(x, None, None, W, f16(-zb), 1e-5, oracle.NORM_NONE,
                            oracle.ACT_SILU, synth.F16)
    np.testing.assert_allclose(yneg[0], y[0] - zb, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ ReLU, GELU
def _act_sweep(act, zb_values, x_rows=2, K=8, seed=18):
    """act(bias) through a zero weight: y[m, n] = act(bias[n]) for every row."""
    bias = f16(zb_values)
    x = f16(np.random.default_rng(seed).normal(0, 1, (x_rows, K)))
    W = f16(np.zeros((len(zb_values), K)))
    y = oracle.norm_gemm(x, None, None, W, bias, 1e-5, oracle.NORM_LAYERNORM, act, synth.F16)
    return y, val16(bias, synth.F16)


def test_relu_closed_form_via_zero_weight_and_bias_sweep():
    y, zb = _act_sweep(oracle.ACT_RELU, np.linspace(-20, 20, 41))
    for m in range(y.shape[0]):
        assert np.array_equal(y[m], np.where(zb < 0, 0.0, zb))
    # ReLU(z) - ReLU(-z) = z
    yn, _ = _act_sweep(oracle.ACT_RELU, -zb)
    np.testing.assert_array_equal(y[0] - yn[0], zb)


def test_gelu_closed_forms_via_zero_weight_and_bias_sweep():
    y, zb = _act_sweep(oracle.ACT_GELU, np.linspace(-8, 8, 33))
    ref = Fn.gelu(t64(zb), approximate="none").numpy()
    for m in range(y.shape[0]):
        np.testing.assert_allclose(y[m], ref, rtol=1e-14, atol=1e-300)
    # GELU(0) = 0; GELU(z) - GELU(-z) = z (Phi(z) + Phi(-z) = 1)
    assert y[0][len(zb) // 2] == 0.0
    yn, _ = _act_sweep(oracle.ACT_GELU, -zb)
    np.testing.assert_allclose(y[0] - yn[0], zb, rtol=1e-14, atol=1e-14)


def test_gelu_at_normal_table_points():
    with open(os.path.join(GOLDEN, "gelu_normal_table.json"), encoding="utf-8") as f:
        gd = json.load(f)
    from scipy.special import ndtr   # an implementation independent of libm's erf
    for z, p in gd["phi"].items():
        assert abs(float(ndtr(float(z))) - p) < 1e-15
        assert abs(1.0 - p - gd["upper_tail"][z]) < 1e-15
    env = {f"phi{z}": p for z, p in gd["phi"].items()}
    env.update({f"tail{z}": p for z, p in gd["upper_tail"].items()})
    ref = np.array([float(eval(s, {"__builtins__": {}}, env)) for s in gd["gelu_expected"]])
    y, _ = _act_sweep(oracle.ACT_GELU, np.array(gd["gelu_of"]))
    np.testing.assert_allclose(y[0], ref, rtol=1e-13, atol=0)


# ------------------------------------------------------------ hand-worked
def _golden():
    with open(os.path.join(GOLDEN, "ln_rms_worked_example.json"), encoding="utf-8") as f:
        return json.load(f)


def _ev(s):
    return float(eval(s, {"__builtins__": {}}, {"sqrt": math.sqrt, "exp": math.exp}))


def test_hand_worked_layernorm_linear_bias():
    gd = _golden()
    x, W, bias = f16(gd["x"]), f16(gd["W"]), f16(gd["bias"])
    y = oracle.norm_gemm(x, None, None, W, bias, gd["eps"], oracle.NORM_LAYERNORM,
                         oracle.ACT_NONE, synth.F16)
    ref = np.array([[_ev(s) for s in row] for row in gd["layernorm_linear_bias"]])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    ys = oracle.norm_gemm(x, None, None, W, bias, gd["eps"], oracle.NORM_LAYERNORM,
                          oracle.ACT_SILU, synth.F16)
    np.testing.assert_allclose(ys, ref / (1 + np.exp(-ref)), rtol=1e-12, atol=1e-12)


def test_hand_worked_rmsnorm_linear():
    gd = _golden()
    x, W = f16(gd["rms_x"]), f16(gd["W"])
    y = oracle.norm_gemm(x, None, None, W, None, gd["eps"], oracle.NORM_RMSNORM,
                         oracle.ACT_NONE, synth.F16)
    ref = np.array([[_ev(s) for s in row] for row in gd["rms_linear_nobias"]])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_hand_worked_silu_values():
    gd = _golden()
    z = np.array([_ev(s) for s in gd["silu_of"]])
    N = len(z)
    y = oracle.norm_gemm(f16(np.zeros((1, 4))), None, None, f16(np.zeros((N, 4))),
                         f16(z), 1e-5, oracle.NORM_NONE, oracle.ACT_SILU, synth.F16)
    ref = np.array([_ev(s) for s in gd["silu_expected"]])
    np.testing.assert_allclose(y[0], ref, rtol=1e-15, atol=0)


# -------------------------------------------------------------------- FFN
@pytest.mark.parametrize("norm,act", [(oracle.NORM_NONE, oracle.ACT_SILU),
                                      (oracle.NORM_LAYERNORM, oracle.ACT_SILU),
                                      (oracle.NORM_LAYERNORM, oracle.ACT_RELU),
                                      (oracle.NORM_RMSNORM, oracle.ACT_GELU)])
def test_ffn_matches_unfused_torch_composition(norm, act):
    """LayerNorm -> MatMul + bias -> act -> MatMul + bias: with ReLU, the chain
    of page 3, section 3.3."""
    rng = np.random.default_rng(16)
    M, K, F, N = 5, 19, 23, 11
    x, g, b = f16(rng.normal(0, 1, (M, K))), f16(rng.normal(1, .3, K)), f16(rng.normal(0, .3, K))
    W1, W2 = f16(rng.normal(0, .3, (F, K))), f16(rng.normal(0, .3, (N, F)))
    b1, b2 = f16(rng.normal(0, .3, F)), f16(rng.normal(0, .3, N))
    y = oracle.ffn(x, g, b, W1, b1, W2, b2, 1e-5, norm, act, synth.F16)
    X = t64(val16(x, synth.F16))
    G, B = t64(val16(g, synth.F16)), t64(val16(b, synth.F16))
    if norm == oracle.NORM_LAYERNORM:
        X = Fn.layer_norm(X, (K,), G, B, float(np.float32(1e-5)))
    elif norm == oracle.NORM_RMSNORM:
        X = Fn.rms_norm(X, (K,), G, float(np.float32(1e-5))) + B
    H = TORCH_ACT[act](Fn.linear(X, t64(val16(W1, synth.F16)), t64(val16(b1, synth.F16))))
    ref = Fn.linear(H, t64(val16(W2, synth.F16)), t64(val16(b2, synth.F16))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("norm,act,bias", [(oracle.NORM_RMSNORM, oracle.ACT_SILU, False),
                                           (oracle.NORM_LAYERNORM, oracle.ACT_GELU, True),
                                           (oracle.NORM_NONE, oracle.ACT_SILU, True)])
def test_gated_ffn_matches_unfused_torch_composition(norm, act, bias):
    """SwiGLU: down(act(gate(a)) * up(a)) with W1 = [W_gate; W_up]."""
    rng = np.random.default_rng(19)
    M, K, F, N = 6, 21, 13, 9
    x, g, b = f16(rng.normal(0, 1, (M, K))), f16(rng.normal(1, .3, K)), f16(rng.normal(0, .3, K))
    W1, W2 = f16(rng.normal(0, .3, (2 * F, K))), f16(rng.normal(0, .3, (N, F)))
    b1 = f16(rng.normal(0, .3, 2 * F)) if bias else None
    b2 = f16(rng.normal(0, .3, N)) if bias else None
    y = oracle.ffn(x, g, b, W1, b1, W2, b2, 1e-5, norm, act, synth.F16, gated=True)
    X = t64(val16(x, synth.F16))
    G, B = t64(val16(g, synth.F16)), t64(val16(b, synth.F16))
    if norm == oracle.NORM_LAYERNORM:
        X = Fn.layer_norm(X, (K,), G, B, float(np.float32(1e-5)))
    elif norm == oracle.NORM_RMSNORM:
        X = Fn.rms_norm(X, (K,), G, float(np.float32(1e-5))) + B
    Wt = t64(val16(W1, synth.F16))
    Bt = t64(val16(b1, synth.F16)) if bias else torch.zeros(2 * F, dtype=torch.float64)
    gate, up = Fn.linear(X, Wt[:F], Bt[:F]), Fn.linear(X, Wt[F:], Bt[F:])
    B2 = t64(val16(b2, synth.F16)) if bias else None
    ref = Fn.linear(TORCH_ACT[act](gate) * up, t64(val16(W2, synth.F16)), B2).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_gated_ffn_with_unit_up_projection_is_the_plain_ffn():
    """W_up = 0 and b_up = 1 make the gate factor 1: the ungated FFN."""
    rng = np.random.default_rng(20)
    M, K, F, N = 5, 16, 11, 7
    x = f16(rng.normal(0, 1, (M, K)))
    Wg, W2 = f16(rng.normal(0, .3, (F, K))), f16(rng.normal(0, .3, (N, F)))
    bg = f16(rng.normal(0, .3, F))
    W1 = np.concatenate([Wg, f16(np.zeros((F, K)))])
    b1 = np.concatenate([bg, f16(np.ones(F))])
    y = oracle.ffn(x, None, None, W1, b1, W2, None, 1e-5, oracle.NORM_NONE, oracle.ACT_SILU,
                   synth.F16, gated=True)
    ref = oracle.ffn(x, None, None, Wg, bg, W2, None, 1e-5, oracle.NORM_NONE, oracle.ACT_SILU,
                     synth.F16)
    np.testing.assert_array_equal(y, ref)


def test_ffn_equals_two_norm_gemm_calls_with_unrounded_h():
    rng = np.random.default_rng(17)
    M, K, F, N = 4, 16, 12, 9
    x = f16(rng.normal(0, 1, (M, K)))
    W1, W2 = f16(rng.normal(0, .3, (F, K))), f16(rng.normal(0, .3, (N, F)))
    y = oracle.ffn(x, None, None, W1, None, W2, None, 1e-5, oracle.NORM_NONE,
                   oracle.ACT_SILU, synth.F16, rows=[3, 1], cols=[8, 0, 4])
    h = oracle.norm_gemm(x, None, None, W1, None, 1e-5, oracle.NORM_NONE,
                         oracle.ACT_SILU, synth.F16)
    ref = h @ val16(W2, synth.F16).T
    np.testing.assert_allclose(y, ref[np.ix_([3, 1], [8, 0, 4])], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ arguments
def test_oracle_rejects_bad_arguments():
    x = f16(np.ones((2, 3)))
    W = f16(np.ones((4, 3)))
    with pytest.raises(ValueError):
        oracle.norm_gemm(x, None, None, W, None, 1e-5, 5, 0, synth.F16)
    with pytest.raises(ValueError):
        oracle.norm_gemm(x, None, None, W, None, 1e-5, 0, 0, synth.F16, rows=[2])
    with pytest.raises(ValueError):
        oracle.norm_gemm(x, None, None, W, None, 1e-5, 0, 0, synth.F16, cols=[4])


def test_epsilon_is_the_float32_value():
    # With a constant-free row of two values the result depends on eps exactly.
    x = f16([[0.0, 2.0]])
    a = oracle.normalize(x, None, None, 1e-1, oracle.NORM_LAYERNORM, synth.F16)
    e32 = float(np.float32(0.1))
    assert a[0, 1] == 1.0 / math.sqrt(1.0 + e32)
