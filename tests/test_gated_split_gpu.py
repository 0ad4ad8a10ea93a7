"""GPU parity of the gated (SwiGLU-style) FFN when its first GEMM's tiles take
more than one round of the CUs and the last round holds at most half of them:
each tile of that round is computed as two halves of its K steps, whose fp32
gate and up sums go to the workspace's [gate | up] area, and a second kernel
forms h = act(gate + b_gate) * (up + b_up) for those tiles (page
"CANN推理加速库ascend-transformer-boost ATB算子融合实战…", Llama2 section: the
FFN's SwiGLU fused with its MatMuls). Every output against the fp64 oracle,
run to run."""
import ctypes

import pytest
import torch

import oracle
import synth
from helpers import assert_close, to_f64, upload

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


def split_tiles(M, F, K):
    import norm_gemm_amd as ng
    lib = ng.lib
    lib.ng_gated_split_tiles.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int]
    lib.ng_gated_split_tiles.restype = ctypes.c_int
    return lib.ng_gated_split_tiles(M, F, K, torch.cuda.get_device_properties(0).multi_processor_count)


# (M, K, F, N, norm, act, dtype, gamma, beta, b1, b2): 288 tiles (32 split,
# prescaled fp16 RMSNorm, SiLU, no biases); 270 tiles of 3 row blocks (the
# last of 44 rows) and 90 column blocks (the last of 108 columns), ragged K
# (264: the second half ends with an 8-element step), bf16 LayerNorm with
# gamma, beta and both biases, GELU
SHAPES = [(512, 320, 9216, 64, RMS, "silu", F16, True, False, False, False),
          (300, 264, 11500, 72, LN, "gelu", BF16, True, True, True, True)]


@pytest.mark.parametrize("M,K,F,N,norm,act,dtype,gamma,beta,b1,b2", SHAPES)
def test_gated_ffn_last_round_split_every_output(M, K, F, N, norm, act, dtype, gamma, beta, b1, b2):
    import norm_gemm_amd as ng
    S = split_tiles(M, F, K)
    if S == 0:
        pytest.skip("the tiles of this shape fill the CUs of this device differently")
    print(f"gated {M}x{K}x{F}x{N}: {S} tiles split", flush=True)
    acts = {"silu": synth.ACT_SILU, "gelu": synth.ACT_GELU}
    case = synth.make_gated_ffn(f"gated_split_{M}x{K}x{F}x{N}", M, K, F, N, dtype=dtype, norm=norm,
                                act=acts[act], gamma=gamma, beta=beta, b1=b1, b2=b2, eps=1e-5,
                                seed=M + F)
    A = case.arrays
    u = lambda k: upload(A.get(k), dtype)
    args = (u("x"), u("W1"), u("W2"), u("gamma"), u("beta"), u("b1"), u("b2"))
    y1 = ng.fused_gated_ffn(*args, eps=1e-5, norm=norm, act=act)
    y2 = ng.fused_gated_ffn(*args, eps=1e-5, norm=norm, act=act)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    err = assert_close(to_f64(y1), ref, what=case.name)
    print(f"{case.name}: every output, max rel err {err:.3e}", flush=True)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
