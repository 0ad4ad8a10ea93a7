"""GPU parity of the skipped-slice split K: a plain GEMM whose 128 x 256 tiles
fill more than half but not all of the CUs keeps one workgroup per tile,
which skips one slice of K steps that a spare CU computes; the two fp32
partial sums are added in a fixed order by a second kernel. It serves the
second GEMM of the FFN (page "昇腾CANN的MatMul融合玩法，让大模型推理快3倍", section 二,
strategy 2) and the GEMM of the post-GEMM normalization (same page, section
五, optimization 3) when their workspace holds two planes of partials.
Compared with the fp64 oracle, run to run, and with the unsplit call."""
import ctypes

import pytest
import torch

import oracle
import synth
from helpers import assert_close, one_ulp, tdtype, tile_indices, to_f64, upload

pytestmark = pytest.mark.gpu

LN, RMS = synth.NORM_LAYERNORM, synth.NORM_RMSNORM
SILU = synth.ACT_SILU
F16, BF16 = synth.F16, synth.BF16


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import norm_gemm_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def skip_plan(M, N, K):
    """(spare workgroups per XCD, slice length) on this device, or None."""
    import norm_gemm_amd as ng
    lib = ng.lib
    ci = ctypes.c_int
    lib.ng_skip_slice_plan.argtypes = [ctypes.c_int64] * 3 + [ci, ctypes.POINTER(ci),
                                                              ctypes.POINTER(ci)]
    lib.ng_skip_slice_plan.restype = ci
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t, ln = ci(0), ci(0)
    return (t.value, ln.value) if lib.ng_skip_slice_plan(M, N, K, cus, t, ln) else None


# (M, K, F, N, dtype, every_row): 144 tiles (3 row blocks, the last of 44
# rows) with a ragged last K step (F = 1800) and two slots, compared in full;
# 224 tiles (the FFN second GEMM's grid of 4 x 56 tiles) with seven slots,
# compared on rows covering every row block and every column
FFN_SHAPES = [(300, 128, 1800, 12288, F16, True), (512, 64, 5376, 14336, BF16, False)]


@pytest.mark.parametrize("M,K,F,N,dtype,every_row", FFN_SHAPES)
def test_ffn_second_gemm_skipped_slice(M, K, F, N, dtype, every_row):
    import norm_gemm_amd as ng
    plan = skip_plan(M, N, F)
    if plan is None:
        pytest.skip("the tiles of this shape fill the CUs of this device differently")
    print(f"ffn {M}x{K}x{F}x{N}: spare workgroups per XCD, slice steps = {plan}", flush=True)
    case = synth.make_ffn(f"ffn_skip_{M}x{K}x{F}x{N}", M, K, F, N, dtype=dtype, norm=LN, act=SILU,
                          gamma=True, beta=True, b1=True, b2=True, seed=M + F)
    A = case.arrays
    u = lambda k: upload(A[k], dtype)
    args = (u("x"), u("W1"), u("W2"), u("gamma"), u("beta"), u("b1"), u("b2"))
    need = ng.fused_ffn_workspace_size(M, F, tdtype(dtype))
    big = torch.empty(need + 8 * M * N, dtype=torch.uint8, device="cuda")
    small = torch.empty(need, dtype=torch.uint8, device="cuda")
    y1 = ng.fused_ffn(*args, eps=1e-5, norm=LN, act="silu", workspace=big)
    y2 = ng.fused_ffn(*args, eps=1e-5, norm=LN, act="silu", workspace=big)
    y0 = ng.fused_ffn(*args, eps=1e-5, norm=LN, act="silu", workspace=small)
    torch.cuda.synchronize()
    rows = list(range(M)) if every_row else tile_indices(M, 128, seed=5, interior=2)
    ref = oracle.run_case(case, rows=None if every_row else rows)
    err = assert_close(to_f64(y1)[rows], ref, what=case.name)
    print(f"{case.name}: {len(rows)} rows x {N} columns, max rel err {err:.3e}", flush=True)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert_close(to_f64(y1), to_f64(y0), tol=one_ulp(dtype), what="skipped slice vs unsplit")
    assert torch.isfinite(y1).all()


def test_ffn_skipped_slice_rewrites_a_used_workspace():
    """Two calls in a row on one workspace, the second with other inputs of
    the same shape: the partial planes are fully rewritten by every call."""
    import norm_gemm_amd as ng
    M, K, F, N = 300, 128, 1800, 12288
    if skip_plan(M, N, F) is None:
        pytest.skip("the tiles of this shape fill the CUs of this device differently")
    need = ng.fused_ffn_workspace_size(M, F, torch.float16)
    big = torch.full((need + 8 * M * N,), 0x7f, dtype=torch.uint8, device="cuda")
    outs = []
    for seed in (3, 4):
        case = synth.make_ffn(f"ffn_skip_reuse_{seed}", M, K, F, N, norm=RMS, act=SILU,
                              gamma=True, beta=False, b1=False, b2=True, seed=seed)
        A = case.arrays
        u = lambda k: upload(A.get(k), F16)
        y = ng.fused_ffn(u("x"), u("W1"), u("W2"), u("gamma"), None, None, u("b2"), eps=1e-5,
                         norm=RMS, act="silu", workspace=big)
        torch.cuda.synchronize()
        rows = tile_indices(M, 128, seed=seed, interior=2)
        assert_close(to_f64(y)[rows], oracle.run_case(case, rows=rows), what=case.name)
        outs.append(y)
    assert not torch.equal(outs[0], outs[1])


def test_gemm_norm_skipped_slice():
    """Post-GEMM LayerNorm whose GEMM makes 144 tiles: the two-plane workspace
    takes the skipped-slice schedule; parity on rows covering every row
    block, run-to-run identity, and agreement with the one-plane call."""
    import norm_gemm_amd as ng
    M, N, K = 300, 12288, 1800
    if skip_plan(M, N, K) is None:
        pytest.skip("the tiles of this shape fill the CUs of this device differently")
    case = synth.make_gemm_norm("gemm_norm_skip", M, K, N, norm=LN, bias=True, gamma=True,
                                beta=True, eps=1e-5, seed=31)
    A = case.arrays
    u = lambda k: upload(A.get(k), F16)
    args = (u("x"), u("W"), u("bias"), u("gamma"), u("beta"))
    plane = ng.fused_gemm_norm_workspace_size(M, N)
    one = torch.empty(plane, dtype=torch.uint8, device="cuda")
    two = torch.empty(2 * plane, dtype=torch.uint8, device="cuda")
    y1 = ng.fused_gemm_norm(*args, eps=1e-5, norm=LN, workspace=one)
    y2 = ng.fused_gemm_norm(*args, eps=1e-5, norm=LN, workspace=two)
    y3 = ng.fused_gemm_norm(*args, eps=1e-5, norm=LN, workspace=two)
    torch.cuda.synchronize()
    rows = tile_indices(M, 128, seed=6, interior=2)
    ref = oracle.run_case(case, rows=rows)
    assert_close(to_f64(y2)[rows], ref, what="two planes")
    assert_close(to_f64(y1)[rows], ref, what="one plane")
    assert torch.equal(y2.view(torch.int16), y3.view(torch.int16))
    assert_close(to_f64(y2), to_f64(y1), tol=one_ulp(F16), what="skipped slice vs unsplit")
