"""GPU parity of the 256 x 192 tiled kernel (page "LayerNorm 融合算子如何让大模型推理
再快 15%？深度拆解 ATB 的实现", sections 2.1-3.2) against the fp64 oracle, and
bit-identity with the 128 x 256 kernel.

The host sends a normalizing call to the wide kernel when 256 x 192 tiles
move fewer bytes per CU over the whole call (ng_wide_tiles_pay on the
device's CU count); the shapes below do on a 256-CU MI355X, with ragged row
and column tiles. Each output element is the same chain of MFMAs in the same k order in
both kernels, with the same normalization arithmetic, so the columns a
narrower call computes on the 128 x 256 kernel must match bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, assert_close, to_f64, upload

pytestmark = pytest.mark.gpu

NONE, LN, RMS = synth.NORM_NONE, synth.NORM_LAYERNORM, synth.NORM_RMSNORM
F16, BF16 = synth.F16, synth.BF16
SILU, RELU, GELU, NOACT = synth.ACT_SILU, synth.ACT_RELU, synth.ACT_GELU, synth.ACT_NONE


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import norm_gemm_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def routes_wide(M, N, K):
    import norm_gemm_amd as ng
    lib = ng.lib
    lib.ng_wide_tiles_pay.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.ng_wide_tiles_fit.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return bool(lib.ng_wide_tiles_fit(M, N, K, 1)) and bool(lib.ng_wide_tiles_pay(M, N, cus))


# (M, N, K, norm, act, dtype, gamma, beta, bias): prescaled fp16 RMSNorm with
# and without gamma, fp32 affine with every gamma / beta combination (fp16 and
# bf16); ragged M (129, 257, 300) and N (last tile 136, 72, 8 columns)
WIDE_SHAPES = [
    (129, 32776, 128, RMS, SILU, F16, True, False, False),
    (300, 21768, 192, LN, RELU, F16, True, True, True),
    (400, 16392, 128, LN, GELU, BF16, False, False, True),
    (257, 21768, 128, RMS, NOACT, BF16, True, False, False),
    (500, 16392, 64, RMS, SILU, F16, False, False, True),
    (200, 32776, 128, LN, NOACT, BF16, False, True, False),
    (384, 21768, 128, LN, SILU, F16, False, False, True),
]


@pytest.mark.parametrize("M,N,K,norm,act,dtype,gamma,beta,bias", WIDE_SHAPES)
def test_wide_tiles_every_output(M, N, K, norm, act, dtype, gamma, beta, bias):
    import norm_gemm_amd as ng
    assert routes_wide(M, N, K)
    case = synth.make_norm_gemm(f"wide_{M}x{N}x{K}_n{norm}a{act}d{dtype}", M, K, N, dtype=dtype,
                                norm=norm, act=act, gamma=gamma, beta=beta, bias=bias, eps=1e-5,
                                seed=M + N + K)
    A = case.arrays
    u = lambda k: upload(A.get(k), dtype)
    y = ng.fused_norm_gemm(u("x"), u("W"), u("gamma"), u("beta"), u("bias"), eps=1e-5, norm=norm,
                           act=act)
    # the first 4096 columns on the 128 x 256 kernel (too few tiles to pay)
    nc = 4096
    assert not routes_wide(M, nc, K)
    y1 = ng.fused_norm_gemm(u("x"), u("W")[:nc].contiguous(), u("gamma"), u("beta"),
                            None if not bias else u("bias")[:nc].contiguous(), eps=1e-5,
                            norm=norm, act=act)
    torch.cuda.synchronize()
    err = assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)
    print(f"{case.name}: max rel err {err:.3e}", flush=True)
    assert torch.equal(y[:, :nc].contiguous().view(torch.int16), y1.view(torch.int16))


def test_wide_tiles_deterministic():
    """Two calls give the same bits."""
    import norm_gemm_amd as ng
    M, N, K = 300, 21768, 128
    case = synth.make_norm_gemm("wide_det", M, K, N, norm=RMS, act=SILU, beta=False, bias=False,
                                eps=1e-6, seed=8)
    A = case.arrays
    u = lambda k: upload(A.get(k), F16)
    y1 = ng.fused_norm_gemm(u("x"), u("W"), u("gamma"), eps=1e-6, norm=RMS, act="silu")
    y2 = ng.fused_norm_gemm(u("x"), u("W"), u("gamma"), eps=1e-6, norm=RMS, act="silu")
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("norm,dtype", [(RMS, F16), (LN, BF16)])
def test_ffn_first_gemm_on_wide_tiles(norm, dtype):
    """An FFN with a normalization prologue and a wide hidden layer: its first
    GEMM (x[300,128] W1[21768,128]) takes the 256 x 192 tiles, writing h and
    its statistics records into the workspace; every output of y against
    the oracle."""
    M, K, F, N = 300, 128, 21768, 256
    assert routes_wide(M, F, K)
    case = synth.make_ffn(f"ffn_wide_{norm}_{dtype}", M, K, F, N, dtype=dtype, norm=norm,
                          act=SILU, gamma=True, beta=norm == LN, b1=True, b2=True, seed=31)
    from helpers import run_case_gpu
    y = run_case_gpu(case)
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)
