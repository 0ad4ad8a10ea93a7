"""Pins of the oracle's inference-mode folding (CPU only).

The folded formulation (gamma in the weights, W' = W * gamma, c1 = W' 1,
c2 = W beta + bias, y = act(r (x W'^T - mu c1) + c2)) is exact algebra of the
unfused definition, so in fp64 it must reproduce oracle.norm_gemm to rounding
noise; its special cases reduce to closed forms and a hand-worked example.
"""
import numpy as np
import pytest

import oracle
import synth

LN, RMS = synth.NORM_LAYERNORM, synth.NORM_RMSNORM


def dec(bits, dtype):
    return oracle.decode(bits, dtype)


@pytest.mark.parametrize("norm", [LN, RMS])
@pytest.mark.parametrize("gamma,beta,bias", [(True, True, True), (True, False, False),
                                             (False, True, True), (False, False, False)])
@pytest.mark.parametrize("dtype,act", [(synth.F16, synth.ACT_SILU), (synth.BF16, synth.ACT_NONE),
                                       (synth.F16, synth.ACT_GELU)])
def test_folded_equals_unfolded_definition(norm, gamma, beta, bias, dtype, act):
    case = synth.make_norm_gemm("fold", 9, 70, 13, dtype=dtype, norm=norm, act=act,
                                gamma=gamma, beta=beta, bias=bias, eps=1e-5, seed=3 + norm)
    A = case.arrays
    Wf, c1, c2 = oracle.fold_weights(A["W"], A["gamma"], A["beta"], A["bias"], dtype)
    got = oracle.norm_gemm_folded(A["x"], Wf, c1, c2, case.eps, norm, act, dtype)
    ref = oracle.run_case(case)
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1.0)) < 1e-12


def test_fold_without_affine_is_the_weight_itself():
    case = synth.make_norm_gemm("fold_id", 2, 33, 7, gamma=False, beta=False, bias=True, seed=5)
    A = case.arrays
    Wf, c1, c2 = oracle.fold_weights(A["W"], None, None, A["bias"], synth.F16)
    W = A["W"].view(np.float16).astype(np.float64)
    assert np.array_equal(Wf, W)
    assert np.allclose(c1, W.sum(axis=1), rtol=0, atol=1e-14)
    assert np.array_equal(c2, A["bias"].view(np.float16).astype(np.float64))


def test_fold_hand_worked_example():
    # W = [[1, 2], [3, -1]], gamma = [2, 0.5], beta = [1, -1], bias = [0.5, 0]:
    # W' = [[2, 1], [6, -0.5]], c1 = [3, 5.5], c2 = [1 - 2 + 0.5, 3 + 1 + 0] = [-0.5, 4]
    f = lambda v: synth.f32_to_f16_bits(np.array(v, dtype=np.float32))
    Wf, c1, c2 = oracle.fold_weights(f([[1, 2], [3, -1]]), f([2, 0.5]), f([1, -1]), f([0.5, 0]),
                                     synth.F16)
    assert np.array_equal(Wf, [[2.0, 1.0], [6.0, -0.5]])
    assert np.array_equal(c1, [3.0, 5.5])
    assert np.array_equal(c2, [-0.5, 4.0])


@pytest.mark.parametrize("act", [synth.ACT_NONE, synth.ACT_SILU])
def test_folded_constant_row_gives_act_of_c2(act):
    """A constant row normalizes to 0 under LayerNorm: r (sum_k c W'_k - c c1)
    vanishes and y = act(W beta + bias) = act(c2)."""
    case = synth.make_norm_gemm("fold_const", 3, 64, 11, norm=LN, act=act, seed=7)
    A = case.arrays
    A["x"] = synth.f32_to_f16_bits(np.full((3, 64), 1.5, dtype=np.float32))
    Wf, c1, c2 = oracle.fold_weights(A["W"], A["gamma"], A["beta"], A["bias"], synth.F16)
    got = oracle.norm_gemm_folded(A["x"], Wf, c1, c2, 1e-5, LN, act, synth.F16)
    z = c2 if act == synth.ACT_NONE else c2 / (1.0 + np.exp(-c2))
    assert np.allclose(got, np.broadcast_to(z, got.shape), rtol=0, atol=1e-9)


def test_folded_large_mean_rows_cancel_in_fp64():
    """x ~ N(1000, 1): x W'^T and mu c1 are ~1000 times the result, and their
    difference still matches the two-pass definition in fp64."""
    case = synth.make_norm_gemm("fold_mean", 4, 512, 9, norm=LN, x_mean=1000.0, seed=9)
    A = case.arrays
    Wf, c1, c2 = oracle.fold_weights(A["W"], A["gamma"], A["beta"], A["bias"], synth.F16)
    got = oracle.norm_gemm_folded(A["x"], Wf, c1, c2, case.eps, LN, 0, synth.F16)
    ref = oracle.run_case(case)
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1.0)) < 1e-9


def test_folded_rejects_no_norm_and_bad_indices():
    case = synth.make_norm_gemm("fold_bad", 2, 8, 3, seed=1)
    A = case.arrays
    Wf, c1, c2 = oracle.fold_weights(A["W"], A["gamma"], A["beta"], A["bias"], synth.F16)
    with pytest.raises(ValueError):
        oracle.norm_gemm_folded(A["x"], Wf, c1, c2, 1e-5, synth.NORM_NONE, 0, synth.F16)
    with pytest.raises(ValueError):
        oracle.norm_gemm_folded(A["x"], Wf, c1, c2, 1e-5, LN, 0, synth.F16, rows=[2])
