"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Acceptance: max |gpu - ref| / (|ref| + 1) <= 1e-2 (fp16/bf16 output, fp32
accumulation), every GPU value finite where the oracle's is; integer GEMMs
must match bit for bit. Small shapes compare every output and span several
tiles with ragged tails; at full size the LayerNorm + Linear layer and the
decode shapes compare every output, the other workloads every output tile
(edges and a seeded interior row and column of each), in the launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (TOL, assert_close, one_ulp, run_case_gpu, tdtype, tile_indices, to_f64,
                     upload)

pytestmark = pytest.mark.gpu

LN, RMS, NONE = synth.NORM_LAYERNORM, synth.NORM_RMSNORM, synth.NORM_NONE
SILU, ACT0 = synth.ACT_SILU, synth.ACT_NONE
F16, BF16 = synth.F16, synth.BF16


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import norm_gemm_amd  # noqa: F401  (fails loudly when the library is missing)
    yield
    torch.cuda.synchronize()


def check_full(case, tol=TOL):
    y = run_case_gpu(case)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    err = assert_close(to_f64(y).reshape(ref.shape), ref, tol, case.name)
    print(f"{case.name}: max rel err {err:.3e}", flush=True)
    return y, ref


# ---------------------------------------------------------------- small shapes
def test_ln_linear_bias_64x256_every_output():
    check_full(synth.ln_linear_bias_64x256())


PREFILL_SHAPES = [(33, 17, 13), (65, 129, 257), (129, 65, 64), (200, 300, 1001),
                  (257, 513, 520), (96, 256, 8), (300, 40, 7)]


@pytest.mark.parametrize("M,N,K", PREFILL_SHAPES)
@pytest.mark.parametrize("norm,act,dtype", [(LN, ACT0, F16), (RMS, SILU, F16), (NONE, SILU, BF16),
                                            (LN, SILU, BF16)])
def test_prefill_ragged_shapes(M, N, K, norm, act, dtype):
    case = synth.make_norm_gemm(f"prefill_{M}x{N}x{K}_n{norm}a{act}d{dtype}", M, K, N,
                                dtype=dtype, norm=norm, act=act, eps=1e-5, seed=M + N + K)
    check_full(case)


DECODE_SHAPES = [(1, 16, 8), (1, 300, 1000), (3, 100, 37), (8, 129, 256), (16, 64, 520),
                 (17, 300, 264), (31, 48, 1001), (32, 1000, 2048)]


@pytest.mark.parametrize("M,N,K", DECODE_SHAPES)
@pytest.mark.parametrize("norm,act,dtype", [(RMS, ACT0, BF16), (LN, SILU, F16), (NONE, ACT0, F16)])
def test_decode_ragged_shapes(M, N, K, norm, act, dtype):
    case = synth.make_norm_gemm(f"decode_{M}x{N}x{K}_n{norm}a{act}d{dtype}", M, K, N,
                                dtype=dtype, norm=norm, act=act, eps=1e-6, seed=M * 7 + N + K)
    check_full(case)


# Aligned decode shapes (K % 8 == 0) that select each slab height of the
# line-streaming decode kernel: 16 * nbk rows of W per workgroup with
# nbk = clamp(ceil(ceil(N / 16) / 256), 2, 8) on a 256-CU device. The K values
# leave a ragged last k-block (K % 64 == 8), idle waves (fewer than 8 k-blocks
# per wave range), odd k-block counts per wave (a tail after the unrolled
# pairs), and the last case needs more workgroups than CUs.
DECODE_SLAB_SHAPES = [
    (1, 9000, 200, RMS, ACT0, BF16, True),      # nbk 3, 4 k-blocks: waves 4..7 idle
    (16, 13000, 136, LN, SILU, F16, True),      # nbk 4
    (17, 17000, 64, NONE, ACT0, BF16, False),   # nbk 5, one k-block: only wave 0 works
    (32, 21000, 520, LN, ACT0, BF16, True),     # nbk 6, 9 k-blocks: wave 4 has one
    (5, 26000, 1096, RMS, SILU, F16, False),    # nbk 7, 3 k-blocks per wave (pair + tail)
    (32, 30000, 2056, RMS, ACT0, F16, True),    # nbk 8, 5 k-blocks per wave
    (9, 40000, 264, LN, SILU, BF16, True),      # nbk 8, 313 workgroups
    # M <= 16 kernel: rows past 8 and rows longer than 8192 take the second
    # statistics pass; N = 17 moves the last 16-row slab back onto row 1
    (12, 2056, 8200, LN, SILU, F16, True),
    (2, 17, 1024, RMS, ACT0, BF16, False),
    (16, 4100, 16384, RMS, SILU, BF16, True),
]


@pytest.mark.parametrize("M,N,K,norm,act,dtype,bias", DECODE_SLAB_SHAPES)
def test_decode_slab_heights(M, N, K, norm, act, dtype, bias):
    case = synth.make_norm_gemm(f"decode_slab_{M}x{N}x{K}", M, K, N, dtype=dtype, norm=norm,
                                act=act, bias=bias, eps=1e-6, seed=M + N // 7 + K)
    check_full(case)


# bf16 RMSNorm without beta on the 16-row-slab kernel (M 17..32) scales after
# the product, with each row's sum of squares taken on the matrix cores:
# ragged K, rows past 8192, idle waves, N below one slab, with and without
# gamma, with SiLU and bias after the scaling
DECODE_LATE_RMS_SHAPES = [
    (17, 9000, 200, True, ACT0, True),
    (24, 13000, 1096, False, SILU, False),
    (32, 21000, 520, True, SILU, True),
    (32, 4100, 16384, True, ACT0, False),
    (20, 17, 1024, False, ACT0, True),
]


@pytest.mark.parametrize("M,N,K,gamma,act,bias", DECODE_LATE_RMS_SHAPES)
def test_decode_late_rms_scaling(M, N, K, gamma, act, bias):
    case = synth.make_norm_gemm(f"decode_late_rms_{M}x{N}x{K}", M, K, N, dtype=BF16, norm=RMS,
                                act=act, gamma=gamma, beta=False, bias=bias, eps=1e-6,
                                seed=M * 3 + N + K)
    check_full(case)


@pytest.mark.parametrize("M", [5, 100])
@pytest.mark.parametrize("gamma,beta,bias", [(False, False, False), (True, False, True),
                                             (False, True, False)])
def test_optional_gamma_beta_bias(M, gamma, beta, bias):
    case = synth.make_norm_gemm(f"opt_{M}_{gamma}{beta}{bias}", M, 136, 72, norm=LN, act=SILU,
                                gamma=gamma, beta=beta, bias=bias, seed=3)
    check_full(case)


@pytest.mark.parametrize("M", [7, 130])
def test_rmsnorm_with_beta(M):
    case = synth.make_norm_gemm(f"rms_beta_{M}", M, 96, 80, norm=RMS, act=ACT0, seed=4)
    check_full(case)


@pytest.mark.parametrize("M,K", [(9, 64), (140, 264)])
def test_unaligned_pointers_take_element_loads(M, K):
    """Pointers that are 2- but not 16-byte aligned must still be exact."""
    case = synth.make_norm_gemm(f"unaligned_{M}x{K}", M, K, 50, norm=LN, act=SILU, seed=5)
    import norm_gemm_amd as ng
    A = case.arrays

    def shifted(bits):
        t = upload(bits, case.dtype)
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    y = ng.fused_norm_gemm(shifted(A["x"]), shifted(A["W"]), shifted(A["gamma"]),
                           shifted(A["beta"]), shifted(A["bias"]), eps=case.eps, norm=LN, act=SILU)
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), what=case.name)


def test_stress_large_mean_layernorm():
    """x ~ N(4, 1): the one-pass fp32 variance must not cancel."""
    for M in (20, 150):
        case = synth.make_norm_gemm(f"shifted_mean_{M}", M, 4096, 96, norm=LN, act=ACT0,
                                    x_mean=4.0, seed=6)
        check_full(case)


# --------------------------------------------------------- closed forms / exact
@pytest.mark.parametrize("M,dtype", [(12, F16), (77, F16), (20, BF16), (200, BF16)])
def test_identity_weight_returns_normalized_rows(M, dtype):
    import norm_gemm_amd as ng
    K = 256
    case = synth.make_norm_gemm(f"identity_{M}", M, K, K, dtype=dtype, norm=LN, seed=7,
                                bias=False)
    eye = np.eye(K, dtype=np.float32)
    case.arrays["W"] = synth.bits_from_f32(eye, dtype)
    check_full(case)
    # The products are exact and each sum has one nonzero term, so y is the
    # kernel's own normalized operand: gamma/beta = (1, 0) gives x_hat itself.
    A = case.arrays
    y = ng.fused_norm_gemm(upload(A["x"], dtype), upload(A["W"], dtype), eps=case.eps, norm=LN)
    torch.cuda.synchronize()
    ref = oracle.normalize(A["x"], None, None, case.eps, LN, dtype)
    assert_close(to_f64(y), ref, what="identity, no affine")


@pytest.mark.parametrize("M", [6, 96])
def test_constant_rows_give_act_of_beta_w_plus_bias(M):
    K, N = 512, 64
    case = synth.make_norm_gemm(f"constant_{M}", M, K, N, norm=LN, act=SILU, seed=8)
    c = np.linspace(-3.0, 3.0, M, dtype=np.float32)[:, None] * np.ones((1, K), np.float32)
    case.arrays["x"] = synth.f32_to_f16_bits(c)
    y, ref = check_full(case)
    yb = to_f64(y)
    # The one-pass statistics shift by the row's first element, so the mean of
    # a constant row is exact and a == beta up to the rounding residual of
    # mean * rs (the kernels normalize as x * rs - mean * rs): all rows agree.
    for m in range(1, M):
        assert_close(yb[m], yb[0], tol=2e-3, what=f"constant row {m}")


@pytest.mark.parametrize("M,dtype,K", [(40, F16, 128), (3, F16, 128), (70, BF16, 64), (5, BF16, 64)])
def test_integer_gemm_is_bit_exact(M, dtype, K):
    """norm NONE with integer x and W in [-2, 2]: products and fp32 sums are
    exact and |y| stays within the integers the output type holds exactly."""
    import norm_gemm_amd as ng
    rng = np.random.default_rng(M + K)
    N = 96
    x = rng.integers(-2, 3, (M, K)).astype(np.float32)
    W = rng.integers(-2, 3, (N, K)).astype(np.float32)
    bias = rng.integers(-3, 4, N).astype(np.float32)
    xb, Wb, bb = (synth.bits_from_f32(v, dtype) for v in (x, W, bias))
    y = ng.fused_norm_gemm(upload(xb, dtype), upload(Wb, dtype), bias=upload(bb, dtype), norm=NONE)
    torch.cuda.synchronize()
    ref = oracle.norm_gemm(xb, None, None, Wb, bb, 1e-5, NONE, ACT0, dtype)
    assert np.array_equal(to_f64(y), ref)


@pytest.mark.parametrize("M", [4, 64])
def test_silu_closed_form_and_zero(M):
    import norm_gemm_amd as ng
    K, N = 64, 81
    bias = synth.f32_to_f16_bits(np.linspace(-20, 20, N, dtype=np.float32))
    x = synth.normal_bits(np.random.default_rng(9), (M, K), 0.0, 1.0, F16)
    W0 = np.zeros((N, K), np.uint16)
    y = ng.fused_norm_gemm(upload(x, F16), upload(W0, F16), bias=upload(bias, F16), norm=LN,
                           act="silu")
    y0 = ng.fused_norm_gemm(upload(x, F16), upload(W0, F16), norm=LN, act="silu")
    torch.cuda.synchronize()
    ref = oracle.norm_gemm(x, None, None, W0, bias, 1e-5, LN, SILU, F16)
    assert_close(to_f64(y), ref, what="silu(bias)")
    z = to_f64(y0)
    assert np.all(z == 0.0) and not np.any(np.signbit(z))


# ------------------------------------------------------ ReLU / GELU epilogues
RELU, GELU = synth.ACT_RELU, synth.ACT_GELU

# One shape per kernel: LDS prefill (aligned, M > 32; fp16 and bf16), generic
# prefill (K % 8 != 0), 512-byte-piece decode (M <= 16), line decode
# (M <= 32), element-load decode (K % 8 != 0).
ACT_SHAPES = [(129, 300, 264, LN, F16), (257, 513, 520, RMS, BF16), (65, 129, 257, LN, BF16),
              (8, 1000, 2048, RMS, BF16), (32, 1000, 2048, LN, F16), (3, 100, 37, NONE, F16)]


@pytest.mark.parametrize("act", [RELU, GELU])
@pytest.mark.parametrize("M,N,K,norm,dtype", ACT_SHAPES)
def test_relu_gelu_epilogues(M, N, K, norm, dtype, act):
    case = synth.make_norm_gemm(f"act{act}_{M}x{N}x{K}_n{norm}d{dtype}", M, K, N, dtype=dtype,
                                norm=norm, act=act, eps=1e-5, seed=M + 3 * N + K + act)
    check_full(case)


@pytest.mark.parametrize("M", [4, 64])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_relu_gelu_closed_forms_and_zero(M, act):
    """act(bias) through a zero weight, against the oracle at one fp16 rounding
    (1e-3, ten times tighter than the acceptance bar); act(0) = +0."""
    import norm_gemm_amd as ng
    K, N = 64, 81
    bias = synth.f32_to_f16_bits(np.linspace(-8, 8, N, dtype=np.float32))
    x = synth.normal_bits(np.random.default_rng(9), (M, K), 0.0, 1.0, F16)
    W0 = np.zeros((N, K), np.uint16)
    y = ng.fused_norm_gemm(upload(x, F16), upload(W0, F16), bias=upload(bias, F16), norm=LN,
                           act=act)
    y0 = ng.fused_norm_gemm(upload(x, F16), upload(W0, F16), norm=LN, act=act)
    torch.cuda.synchronize()
    ref = oracle.norm_gemm(x, None, None, W0, bias, 1e-5, LN, ng.ACTS[act], F16)
    assert_close(to_f64(y), ref, tol=1e-3, what=f"{act}(bias)")
    if act == "relu":
        assert np.array_equal(to_f64(y), ref)     # exact: max(z, 0) of an fp16 value
    z = to_f64(y0)
    assert np.all(z == 0.0) and not np.any(np.signbit(z))


# ------------------------------------------- persistent tiles / statistics reuse
@pytest.mark.parametrize("M,N,K,norm", [
    (256, 34816, 64, LN),     # 2 x 136 tiles: XCD-grouped, two rounds, stats reused
    (384, 23040, 72, RMS),    # 3 x 90 tiles: plain round-robin, stats recomputed, K tail
    (160, 2056, 200, LN),     # ragged M, N % 8 == 0 but N % 256 != 0, K tail
])
def test_persistent_tile_walks(M, N, K, norm):
    case = synth.make_norm_gemm(f"persistent_{M}x{N}x{K}", M, K, N, norm=norm, act=SILU,
                                seed=M + K)
    y = run_case_gpu(case)
    torch.cuda.synchronize()
    rows = tile_indices(M, 128, seed=3)
    cols = tile_indices(N, 256, seed=4)
    ref = oracle.run_case(case, rows=rows, cols=cols)
    assert_close(to_f64(y)[np.ix_(rows, cols)], ref, what=case.name)
    assert torch.isfinite(y).all()


# ------------------------------------------------------------- run properties
@pytest.mark.parametrize("M", [8, 200])
def test_deterministic_and_guard_bands_untouched(M):
    import norm_gemm_amd as ng
    case = synth.make_norm_gemm(f"det_{M}", M, 1024, 384, norm=RMS, act=SILU, seed=10)
    A = case.arrays
    args = [upload(A[k], F16) for k in ("x", "W", "gamma", "beta", "bias")]
    pad = 4096
    buf = torch.full((M * 384 + 2 * pad,), float("nan"), dtype=torch.float16, device="cuda")
    out = buf[pad:pad + M * 384].view(M, 384)
    ng.fused_norm_gemm(args[0], args[1], *args[2:], eps=case.eps, norm=RMS, act="silu", out=out)
    y2 = ng.fused_norm_gemm(args[0], args[1], *args[2:], eps=case.eps, norm=RMS, act="silu")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), y2.view(torch.int16))
    assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[pad + M * 384:]).all()
    assert torch.isfinite(out).all()


def test_decode_rows_are_independent():
    """Row m of an M=32 call equals an M=1 call on that row."""
    import norm_gemm_amd as ng
    case = synth.make_norm_gemm("rows", 32, 2048, 640, dtype=BF16, norm=RMS, bias=False,
                                beta=False, eps=1e-6, seed=11)
    A = case.arrays
    x, W, g = upload(A["x"], BF16), upload(A["W"], BF16), upload(A["gamma"], BF16)
    y = ng.fused_norm_gemm(x, W, g, eps=1e-6, norm=RMS)
    perm = torch.randperm(32, generator=torch.Generator().manual_seed(0)).to("cuda")
    yp = ng.fused_norm_gemm(x[perm].contiguous(), W, g, eps=1e-6, norm=RMS)
    rows = [ng.fused_norm_gemm(x[m:m + 1].contiguous(), W, g, eps=1e-6, norm=RMS) for m in (0, 17, 31)]
    torch.cuda.synchronize()
    for r, m in zip(rows, (0, 17, 31)):
        assert_close(to_f64(r)[0], to_f64(y)[m], what=f"row {m}")
    assert torch.equal(yp.view(torch.int16), y[perm].view(torch.int16))


# -------------------------------------------------------------------- FFN
@pytest.mark.parametrize("M,K,F,N,norm", [(5, 64, 96, 40, NONE), (70, 136, 200, 72, NONE),
                                          (33, 72, 130, 33, LN), (2, 40, 24, 16, RMS)])
def test_ffn_small(M, K, F, N, norm):
    case = synth.make_ffn(f"ffn_{M}x{K}x{F}x{N}", M, K, F, N, norm=norm, gamma=norm != NONE,
                          beta=norm == LN, b1=True, b2=True, seed=12)
    check_full(case)


@pytest.mark.parametrize("M,K,F,N,norm,act", [(33, 72, 130, 33, LN, RELU),
                                              (100, 264, 520, 136, LN, RELU),
                                              (20, 136, 200, 72, RMS, GELU),
                                              (70, 256, 384, 128, NONE, GELU)])
def test_ffn_chain_norm_bias_act(M, K, F, N, norm, act):
    """LayerNorm -> MatMul + bias -> ReLU -> MatMul + bias (the chain of page
    3, section 3.3) and its RMSNorm / GELU variants through fused_ffn."""
    case = synth.make_ffn(f"ffn_chain_{M}x{K}x{F}x{N}_n{norm}a{act}", M, K, F, N, norm=norm,
                          act=act, gamma=norm != NONE, beta=norm == LN, b1=True, b2=True,
                          seed=M + K + F + N)
    check_full(case)


# Gated (SwiGLU-style) FFN: tiles that hold the gate and up rows of the same
# columns (M > 32, aligned; ragged M, F and K; F % 8 != 0 takes the in-kernel
# statistics; several row and column blocks, XCD-grouped), and the
# projections + gating kernel path (M <= 32, K % 8 != 0).
GATED_SHAPES = [
    (70, 136, 200, 72, LN, SILU, F16),
    (129, 264, 384, 136, RMS, SILU, F16),
    (257, 520, 1000, 256, NONE, GELU, BF16),
    (200, 64, 130, 40, LN, RELU, F16),
    (300, 1024, 2048, 512, RMS, SILU, F16),
    (16, 128, 320, 96, RMS, SILU, BF16),
    (5, 264, 136, 48, NONE, GELU, F16),
    (33, 37, 50, 20, LN, SILU, F16),
]


@pytest.mark.parametrize("M,K,F,N,norm,act,dtype", GATED_SHAPES)
def test_gated_ffn(M, K, F, N, norm, act, dtype):
    case = synth.make_gated_ffn(f"gated_ffn_{M}x{K}x{F}x{N}_n{norm}a{act}d{dtype}", M, K, F, N,
                                dtype=dtype, norm=norm, act=act, gamma=norm != NONE,
                                beta=norm == LN, b1=True, b2=True, seed=M + K + F + N)
    check_full(case)


@pytest.mark.parametrize("M", [8, 100])
def test_stacked_qkv_weight_equals_three_calls(M):
    """One RMSNorm output feeding the Q, K and V projections (grouped K/V
    heads) through one call on the stacked [Wq; Wk; Wv] weight: equal to the
    three separate calls, bit for bit on the tiled path (the arithmetic of an
    output element does not depend on N), within tolerance of the oracle."""
    import norm_gemm_amd as ng
    K, NQ, NKV = 512, 512, 128
    case = synth.make_norm_gemm(f"qkv_{M}", M, K, NQ + 2 * NKV, norm=RMS, beta=False,
                                bias=False, eps=1e-5, seed=21 + M)
    A = case.arrays
    x, g, W = upload(A["x"], F16), upload(A["gamma"], F16), upload(A["W"], F16)
    y = ng.fused_norm_gemm(x, W, g, eps=1e-5, norm=RMS)
    parts = [ng.fused_norm_gemm(x, W[a:b].contiguous(), g, eps=1e-5, norm=RMS)
             for a, b in ((0, NQ), (NQ, NQ + NKV), (NQ + NKV, NQ + 2 * NKV))]
    torch.cuda.synchronize()
    joined = torch.cat(parts, dim=1)
    assert_close(to_f64(y), oracle.run_case(case), what="stacked qkv")
    if M > 32:
        assert torch.equal(y.view(torch.int16), joined.view(torch.int16))
    else:
        assert_close(to_f64(joined), to_f64(y), tol=2e-3, what="qkv parts")


@pytest.mark.parametrize("norm,beta,dtype", [(LN, True, F16), (RMS, True, F16), (RMS, False, F16),
                                               (LN, True, BF16), (RMS, False, BF16)])
def test_output_columns_do_not_depend_on_n(norm, beta, dtype):
    """The arithmetic of an output element does not depend on N (tile count,
    statistics records per tile): the first 256 columns of a 768-column call
    equal a call on those 256 rows of W bit for bit."""
    import norm_gemm_amd as ng
    M, K, N = 100, 520, 768
    case = synth.make_norm_gemm(f"onecol_{norm}{beta}{dtype}", M, K, N, dtype=dtype, norm=norm,
                                beta=beta, bias=True, eps=1e-5, seed=77 + norm)
    A = case.arrays
    u = lambda k: upload(A.get(k), dtype)
    x, g, b, W, bias = u("x"), u("gamma"), u("beta"), u("W"), u("bias")
    y = ng.fused_norm_gemm(x, W, g, b, bias, eps=1e-5, norm=norm)
    y1 = ng.fused_norm_gemm(x, W[:256].contiguous(), g, b, bias[:256].contiguous(), eps=1e-5,
                            norm=norm)
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), what="768 columns")
    assert torch.equal(y[:, :256].contiguous().view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("M,K,F,N,dtype", [(100, 264, 520, 136, F16), (300, 512, 2000, 512, BF16),
                                            (64, 136, 200, 72, F16)])
def test_ffn_split_k_of_the_second_gemm(M, K, F, N, dtype):
    """A workspace with room for two fp32 partial sums of y splits the second
    GEMM's K over two workgroups per tile (its tiles fill under half of the
    CUs; F = 200 leaves a ragged last step in the second range): parity
    with the oracle, run-to-run identical, and close to the unsplit call."""
    import norm_gemm_amd as ng
    case = synth.make_ffn(f"ffn_splitk_{M}x{K}x{F}x{N}", M, K, F, N, dtype=dtype, norm=LN,
                          act=SILU, gamma=True, beta=True, b1=True, b2=True, seed=M + F)
    A = case.arrays
    u = lambda k: upload(A[k], dtype)
    args = (u("x"), u("W1"), u("W2"), u("gamma"), u("beta"), u("b1"), u("b2"))
    need = ng.fused_ffn_workspace_size(M, F, tdtype(dtype))
    big = torch.empty(need + 8 * M * N + 4096, dtype=torch.uint8, device="cuda")
    y1 = ng.fused_ffn(*args, eps=1e-5, norm=LN, act="silu", workspace=big)
    y2 = ng.fused_ffn(*args, eps=1e-5, norm=LN, act="silu", workspace=big)
    small = torch.empty(need, dtype=torch.uint8, device="cuda")    # h only: unsplit
    y0 = ng.fused_ffn(*args, eps=1e-5, norm=LN, act="silu", workspace=small)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    assert_close(to_f64(y1), ref, what=case.name)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert_close(to_f64(y1), to_f64(y0), tol=one_ulp(dtype), what="split vs unsplit")


@pytest.mark.parametrize("M", [16, 100])
def test_ffn_equals_two_norm_gemm_calls(M):
    import norm_gemm_amd as ng
    case = synth.make_ffn(f"ffn_compose_{M}", M, 128, 320, 96, norm=LN, gamma=True, beta=True,
                          b1=True, b2=True, seed=13)
    A = case.arrays
    u = lambda k: upload(A[k], F16)
    # a workspace that holds h only: the second GEMM is one unsplit call
    ws = torch.empty(ng.fused_ffn_workspace_size(M, 320, torch.float16), dtype=torch.uint8,
                     device="cuda")
    y = ng.fused_ffn(u("x"), u("W1"), u("W2"), u("gamma"), u("beta"), u("b1"), u("b2"),
                     eps=1e-5, norm=LN, act="silu", workspace=ws)
    h = ng.fused_norm_gemm(u("x"), u("W1"), u("gamma"), u("beta"), u("b1"), eps=1e-5, norm=LN,
                           act="silu")
    y2 = ng.fused_norm_gemm(h, u("W2"), bias=u("b2"), norm=NONE)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


# ----------------------------------------------------------- full-size workloads
# The workloads at their full sizes, in the launch configuration the benchmark
# times. The LayerNorm + Linear layer and the decode shapes are compared in
# full; the others on every output tile: both edges and a seeded interior
# row of every 128-row block, and both edges and a seeded interior column of
# every 256-column block (the tiled kernels' 128 x 256 output tiles).
def check_tiles(case, row_tile=128, col_tile=256, interior=1):
    y = run_case_gpu(case)
    torch.cuda.synchronize()
    rows = tile_indices(case.M, row_tile, seed=1, interior=interior)
    cols = tile_indices(case.N, col_tile, seed=2, interior=interior)
    ref = oracle.run_case(case, rows=rows, cols=cols)
    got = to_f64(y)[np.ix_(rows, cols)]
    err = assert_close(got, ref, what=case.name)
    print(f"{case.name}: {len(rows)} rows x {len(cols)} cols covering every "
          f"{row_tile}x{col_tile} tile, max rel err {err:.3e}", flush=True)
    assert torch.isfinite(y).all()


def test_full_ln_linear_bias_1024x8192_every_output():
    check_full(synth.ln_linear_bias_1024x8192())


@pytest.mark.parametrize("M", [1, 8, 32])
def test_full_decode_rms_gemm_8192x28672_every_output(M):
    check_full(synth.decode_rms_gemm_8192x28672(M))


def test_full_rms_matmul_silu_512x14336():
    check_tiles(synth.rms_matmul_silu_512x14336())


def test_full_ffn_silu_512x14336x49152():
    check_tiles(synth.ffn_silu_512x14336x49152())


def test_ffn_chain_ln_relu_bias_1024x8192():
    """The page-3 chain at its example's width: x[8 x 128, 8192], LayerNorm,
    MatMul 8192 -> 8192 + bias, ReLU, MatMul 8192 -> 8192 + bias."""
    case = synth.make_ffn("ffn_chain_ln_relu_x1024x8192_w1_8192_w2_8192_f16", 1024, 8192, 8192,
                          8192, norm=LN, act=RELU, gamma=True, beta=True, b1=True, b2=True,
                          seed=0)
    check_tiles(case)


def test_gated_ffn_swiglu_rms_512x8192x28672():
    """SwiGLU FFN of the LLaMA-2-70B layer: RMSNorm, [gate; up] 2 x 28672 x 8192,
    down 8192 x 28672, fp16."""
    check_tiles(synth.gated_ffn_swiglu_512x8192x28672())


def test_unaligned_matmul_silu_513x14337():
    """The pages' unaligned shape (page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍",
    section 五, optimization 1): x[513, 14337] . W[49152, 14337]^T + SiLU in
    fp16. K % 8 != 0 takes the generic tiled kernel (128 x 128 tiles); M = 513
    leaves a one-row last block."""
    case = synth.make_norm_gemm("matmul_silu_x513x14337_w49152x14337_f16", 513, 14337, 49152,
                                norm=NONE, act=SILU, gamma=False, beta=False, bias=False, seed=0)
    check_tiles(case, row_tile=128, col_tile=128)


@pytest.mark.parametrize("norm", [NONE, RMS])
def test_unaligned_k14337_small_n_every_output(norm):
    """K = 14337 at a width the oracle computes in full (ragged last K chunk,
    ragged row and column blocks)."""
    case = synth.make_norm_gemm(f"k14337_x513_w300_n{norm}", 513, 14337, 300, norm=norm,
                                act=SILU, beta=False, bias=False, eps=1e-6, seed=1 + norm)
    check_full(case)


# ---------------------------------------------- extreme rows (fp16 statistics)
def _extreme_rows(M, K, seed):
    """fp16 rows that stress the statistics: rows whose 1/sigma far exceeds the
    fp16 range (values a few subnormal steps apart), rows spanning +-40000
    (differences beyond the fp16 range), and ordinary rows between them."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    tiny = np.float32(2.0 ** -24)
    for m in range(M):
        kind = m % 3
        if kind == 0:
            x[m] = rng.integers(-3, 4, K).astype(np.float32) * tiny
        elif kind == 1:
            x[m] = np.where(rng.random(K) < 0.5, -40000.0, 40000.0).astype(np.float32) \
                + rng.standard_normal(K).astype(np.float32) * 100.0
    return synth.f32_to_f16_bits(x)


@pytest.mark.parametrize("M,K", [(6, 512), (12, 1001), (20, 1000), (96, 512), (150, 2056),
                                 (40, 263)])
def test_fp16_layernorm_extreme_rows_eps0(M, K):
    """eps = 0: sigma ~ 1e-7 gives 1/sigma ~ 1e7, beyond fp16, and rows of
    +-40000 make x - x[0] exceed the fp16 range; the statistics and the
    normalization run in fp32, so every path must still match the oracle.
    Covers the skinny kernels (M <= 32, aligned and K % 8 != 0), the tiled
    kernel and the generic tiled kernel (K % 8 != 0)."""
    case = synth.make_norm_gemm(f"extreme_rows_{M}x{K}", M, K, 72, norm=LN, act=ACT0, eps=0.0,
                                seed=M + K)
    case.arrays["x"] = _extreme_rows(M, K, seed=M)
    check_full(case)


@pytest.mark.parametrize("M,K,gamma,eps", [(96, 512, True, 0.0), (150, 2056, False, 0.0),
                                            (40, 264, True, 1e-6), (300, 1024, True, 1e-5)])
def test_fp16_rmsnorm_prescale_extreme_rows(M, K, gamma, eps):
    """fp16 RMSNorm without beta on the tiled kernel scales each row by a
    power of two 2^e <= 1/rms before the single fp16 rounding, with e clamped
    to -14..15, and rescales the fp32 sum by rs 2^-e: rows whose 1/rms is ~1e7
    (clamped at 2^15), rows of +-40000 (clamped at 2^-14) and ordinary rows
    must all match the oracle."""
    case = synth.make_norm_gemm(f"rms_prescale_{M}x{K}_g{gamma}", M, K, 72, norm=RMS, act=SILU,
                                gamma=gamma, beta=False, eps=eps, seed=M + K)
    case.arrays["x"] = _extreme_rows(M, K, seed=M + 1)
    check_full(case)


@pytest.mark.parametrize("M", [40, 130])
def test_gated_ffn_rmsnorm_prescale(M):
    """The gated tiles take the same prescaled operand and rescale both the
    gate and the up sums of a row before act(gate) * up."""
    case = synth.make_gated_ffn(f"gated_prescale_{M}", M, 264, 384, 136, norm=RMS, act=SILU,
                                gamma=True, beta=False, b1=True, b2=True, eps=1e-6, seed=M)
    case.arrays["x"] = _extreme_rows(M, 264, seed=M + 2)
    check_full(case)


@pytest.mark.parametrize("M", [24, 200])
def test_large_mean_layernorm_k14336_tight(M):
    """x ~ N(4, 1) at K = 14336 with gamma and beta: the fp32 normalization is
    rounded once to fp16, so the error stays near one fp16 rounding of the
    operand and the output (pinned at 3e-3, a third of the acceptance bar)."""
    case = synth.make_norm_gemm(f"large_mean_tight_{M}", M, 14336, 256, norm=LN, act=ACT0,
                                x_mean=4.0, eps=1e-5, seed=40 + M)
    check_full(case, tol=3e-3)
