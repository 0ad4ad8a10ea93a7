"""GPU parity of the inference-mode folding (page "LayerNorm 融合算子如何让大模型推理
再快 15%？深度拆解 ATB 的实现", section 6.2, tip 2) against the fp64 oracle.

norm_gemm_fold_weights: W' must equal the round-to-nearest-even of the
oracle's exact W * gamma bit for bit (the product of two 16-bit values is
exact in fp32 and fp64); c1 must be the sum of those rounded values and c2 =
W beta + bias, to fp32 summation accuracy. fused_norm_gemm_folded: the output
against the unfolded definition (oracle.norm_gemm) under the acceptance bar
max |gpu - ref| / (|ref| + 1) <= 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, assert_close, tile_indices, to_f64, upload

pytestmark = pytest.mark.gpu

LN, RMS = synth.NORM_LAYERNORM, synth.NORM_RMSNORM
F16, BF16 = synth.F16, synth.BF16


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import norm_gemm_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def rne16(v, dtype):
    """Round fp64 values to fp16 / bf16 (RNE) with a library routine."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float64))
    return t.to(torch.float16 if dtype == F16 else torch.bfloat16).to(torch.float64).numpy()


def fold_case(case):
    import norm_gemm_amd as ng
    A = case.arrays
    u = lambda k: upload(A.get(k), case.dtype)
    wf, c1, c2 = ng.norm_gemm_fold_weights(u("W"), u("gamma"), u("beta"), u("bias"))
    return u, wf, c1, c2


@pytest.mark.parametrize("N,K,dtype,gamma,beta,bias", [
    (40, 264, F16, True, True, True), (33, 1001, F16, True, False, True),
    (17, 72, BF16, True, True, False), (64, 520, BF16, False, True, True),
    (5, 9, F16, False, False, False)])
def test_fold_weights_bits_and_vectors(N, K, dtype, gamma, beta, bias):
    case = synth.make_norm_gemm(f"fold_{N}x{K}", 2, K, N, dtype=dtype, gamma=gamma, beta=beta,
                                bias=bias, seed=N + K)
    _, wf, c1, c2 = fold_case(case)
    torch.cuda.synchronize()
    A = case.arrays
    Wf, r1, r2 = oracle.fold_weights(A["W"], A["gamma"], A["beta"], A["bias"], dtype)
    want = rne16(Wf, dtype)
    assert np.array_equal(to_f64(wf), want)
    assert np.allclose(to_f64(c1), want.sum(axis=1), rtol=1e-5, atol=1e-5)
    assert np.allclose(to_f64(c2), r2, rtol=1e-5, atol=1e-5)


def check_folded(case, rows=None, cols=None, tol=TOL):
    import norm_gemm_amd as ng
    u, wf, c1, c2 = fold_case(case)
    y = ng.fused_norm_gemm_folded(u("x"), wf, c1 if case.norm == LN else None, c2, eps=case.eps,
                                  norm=case.norm, act=case.act)
    torch.cuda.synchronize()
    ref = oracle.run_case(case, rows=rows, cols=cols)
    got = to_f64(y)
    if rows is not None:
        got = got[np.ix_(rows, cols)]
    err = assert_close(got, ref, tol, case.name)
    print(f"{case.name}: max rel err {err:.3e}", flush=True)
    return err


# tiled kernel at several M (also M <= 32), ragged M / N / K tails (K % 64
# != 0), N % 8 != 0 (statistics in the kernel), LN and RMS, each activation
FOLDED_SHAPES = [(129, 300, 264, LN, synth.ACT_SILU, F16), (257, 513, 520, RMS, synth.ACT_NONE, BF16),
                 (5, 256, 136, LN, synth.ACT_GELU, F16), (32, 100, 72, RMS, synth.ACT_SILU, F16),
                 (200, 81, 1024, LN, synth.ACT_RELU, BF16), (300, 1024, 2056, RMS, synth.ACT_SILU, F16)]


@pytest.mark.parametrize("M,N,K,norm,act,dtype", FOLDED_SHAPES)
def test_folded_gemm_every_output(M, N, K, norm, act, dtype):
    case = synth.make_norm_gemm(f"folded_{M}x{N}x{K}_n{norm}", M, K, N, dtype=dtype, norm=norm,
                                act=act, beta=norm == LN, bias=True, eps=1e-5, seed=M + N + K)
    check_folded(case)


def test_folded_rms_matmul_silu_512x14336():
    """The RMSNorm + MatMul + SiLU workload with folded weights, every
    128 x 256 output tile covered."""
    case = synth.rms_matmul_silu_512x14336()
    check_folded(case, rows=tile_indices(case.M, 128, 1), cols=tile_indices(case.N, 256, 2))


def test_folded_ln_linear_bias_1024x8192_every_output():
    check_folded(synth.ln_linear_bias_1024x8192())


@pytest.mark.parametrize("M", [40, 200])
def test_folded_large_mean_layernorm_stress(M):
    """x ~ N(4, 1) at K = 14336: x W'^T and mu c1 are four times the centred
    sum and cancel in fp32; the result still meets the acceptance bar (the
    normalized-operand path is the accurate choice for larger |mean| / sigma)."""
    case = synth.make_norm_gemm(f"folded_mean4_{M}", M, 14336, 256, norm=LN, x_mean=4.0,
                                eps=1e-5, seed=50 + M)
    check_folded(case)


def test_folded_is_deterministic():
    import norm_gemm_amd as ng
    case = synth.make_norm_gemm("folded_det", 150, 1024, 384, norm=LN, act=synth.ACT_SILU, seed=3)
    u, wf, c1, c2 = fold_case(case)
    y1 = ng.fused_norm_gemm_folded(u("x"), wf, c1, c2, eps=1e-5, norm=LN, act="silu")
    y2 = ng.fused_norm_gemm_folded(u("x"), wf, c1, c2, eps=1e-5, norm=LN, act="silu")
    wf2, c12, c22 = ng.norm_gemm_fold_weights(u("W"), u("gamma"), u("beta"), u("bias"))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(wf.view(torch.int16), wf2.view(torch.int16))
    assert torch.equal(c1, c12) and torch.equal(c2, c22)


@pytest.mark.parametrize("norm", [LN, RMS])
def test_folded_output_columns_do_not_depend_on_n(norm):
    """The first 256 columns of a 640-column folded call equal a call on those
    rows of W', c1 and c2 bit for bit (an output element's arithmetic does not
    depend on N)."""
    import norm_gemm_amd as ng
    case = synth.make_norm_gemm(f"folded_onecol_{norm}", 90, 264, 640, norm=norm,
                                beta=norm == LN, bias=True, eps=1e-5, seed=91 + norm)
    u, wf, c1, c2 = fold_case(case)
    c1 = c1 if norm == LN else None
    y = ng.fused_norm_gemm_folded(u("x"), wf, c1, c2, eps=1e-5, norm=norm)
    y1 = ng.fused_norm_gemm_folded(u("x"), wf[:256].contiguous(),
                                   None if c1 is None else c1[:256].contiguous(),
                                   c2[:256].contiguous(), eps=1e-5, norm=norm)
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)
    assert torch.equal(y[:, :256].contiguous().view(torch.int16), y1.view(torch.int16))


def test_folded_unaligned_is_unsupported():
    import norm_gemm_amd as ng
    case = synth.make_norm_gemm("folded_unaligned", 40, 64, 32, norm=RMS, seed=4)
    u, wf, c1, c2 = fold_case(case)
    x = u("x")
    buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
    xs = buf[1:].view(x.shape)
    xs.copy_(x)
    with pytest.raises(ng.NormGemmError) as e:
        ng.fused_norm_gemm_folded(xs, wf, None, c2, norm="rmsnorm")
    assert e.value.status == -7
