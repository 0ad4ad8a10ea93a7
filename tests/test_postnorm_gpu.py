"""GPU parity of the post-GEMM normalization (page "昇腾CANN的MatMul融合玩法，让大模型
推理快3倍", section 五, optimization 3: the fused MatMul(Output)_RMSNorm) against
the fp64 oracle: every output of ragged shapes (M below and above one tile,
K % 64 != 0, N not a multiple of the tile), LayerNorm and RMSNorm with and
without bias / gamma / beta, the split-K path, and the LLaMA-2-70B attention
output projection at full size."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, assert_close, one_ulp, run_case_gpu, to_f64, upload

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


def check(case, tol=TOL):
    y = run_case_gpu(case)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    err = assert_close(to_f64(y), ref, tol, case.name)
    print(f"{case.name}: max rel err {err:.3e}", flush=True)
    return y


SHAPES = [(5, 300, 264, RMS, F16, False, True, False), (130, 520, 1024, LN, F16, True, True, True),
          (257, 136, 72, RMS, BF16, True, False, False), (40, 8200, 136, LN, BF16, False, True, True),
          (300, 1000, 2056, RMS, F16, False, True, False), (1, 64, 64, LN, F16, False, False, False)]


@pytest.mark.parametrize("M,N,K,norm,dtype,bias,gamma,beta", SHAPES)
def test_gemm_norm_every_output(M, N, K, norm, dtype, bias, gamma, beta):
    case = synth.make_gemm_norm(f"gemm_norm_{M}x{N}x{K}_n{norm}d{dtype}", M, K, N, dtype=dtype,
                                norm=norm, bias=bias, gamma=gamma, beta=beta, eps=1e-5,
                                seed=M + N + K)
    check(case)


def test_gemm_norm_split_k_matches_unsplit():
    """Two fp32 planes split K over two workgroups per tile (the tiles fill
    under half of the CUs): parity, run-to-run identity, and agreement with
    the one-plane call to fp32 summation order."""
    import norm_gemm_amd as ng
    case = synth.make_gemm_norm("gemm_norm_split", 200, 2048, 512, norm=LN, bias=True, beta=True,
                                seed=9)
    A = case.arrays
    u = lambda k: upload(A.get(k), F16)
    args = (u("x"), u("W"), u("bias"), u("gamma"), u("beta"))
    plane = ng.fused_gemm_norm_workspace_size(200, 512)
    one = torch.empty(plane, dtype=torch.uint8, device="cuda")
    two = torch.empty(2 * plane, dtype=torch.uint8, device="cuda")
    y1 = ng.fused_gemm_norm(*args, eps=1e-5, norm=LN, workspace=one)
    y2 = ng.fused_gemm_norm(*args, eps=1e-5, norm=LN, workspace=two)
    y3 = ng.fused_gemm_norm(*args, eps=1e-5, norm=LN, workspace=two)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    assert_close(to_f64(y1), ref, what="one plane")
    assert_close(to_f64(y2), ref, what="two planes")
    assert torch.equal(y2.view(torch.int16), y3.view(torch.int16))
    assert_close(to_f64(y2), to_f64(y1), tol=one_ulp(F16), what="split vs unsplit")


def test_attn_out_rmsnorm_512x8192_every_output():
    check(synth.attn_out_rmsnorm_512x8192())


def test_gemm_norm_rms_invariant_on_gpu():
    """With gamma = 1 and no beta each output row has mean square
    ms / (ms + eps) (here ~1), up to the fp16 rounding of y."""
    case = synth.make_gemm_norm("gemm_norm_inv", 64, 512, 1024, norm=RMS, gamma=False, seed=4)
    y = to_f64(run_case_gpu(case))
    torch.cuda.synchronize()
    assert np.allclose((y * y).mean(axis=1), 1.0, atol=2e-3)


@pytest.mark.parametrize("M,N,K,dtype,offset", [(33, 1001, 200, F16, 0), (3, 16400, 72, BF16, 0),
                                               (70, 2048, 136, F16, 1), (9, 12288, 64, BF16, 0)])
def test_gemm_norm_row_kernel_forms(M, N, K, dtype, offset):
    """The row kernel's forms: rows held in registers with 8-byte accesses
    (N % 4 == 0, N <= 16384), the same with 2-byte accesses (bias, gamma and
    beta at an odd element offset), N % 4 != 0 and N > 16384 (rows re-read
    from L2); LayerNorm with every affine term, every output."""
    import norm_gemm_amd as ng
    case = synth.make_gemm_norm(f"gemm_norm_form_{M}x{N}x{K}_{offset}", M, K, N, dtype=dtype,
                                norm=LN, bias=True, gamma=True, beta=True, eps=1e-5, seed=N + K)
    A = case.arrays

    def vec(k):
        t = upload(A[k], dtype)
        if not offset:
            return t
        buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=t.device)
        buf[offset:] = t
        return buf[offset:]

    y = ng.fused_gemm_norm(upload(A["x"], dtype), upload(A["W"], dtype), vec("bias"),
                           vec("gamma"), vec("beta"), eps=1e-5, norm=LN)
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)
