"""The allocation-free FFN entry point against fused_ffn, through the C ABI.

fused_ffn_noalloc keeps h (and the split-K partials when they fit) in the
library's static per-device array; with a caller workspace of the same size
fused_ffn makes the same kernel choices, so the outputs must be identical.
Two calls in a row, the second smaller, show that the reused array carries
nothing from one call to the next; both also meet the oracle's bar."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, tile_indices, to_f64, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


# The first shape's second GEMM makes 144 tiles (more than half of 256 CUs),
# so it takes the skipped-slice split K with its two fp32 partial planes in
# the scratch past h (compared with the oracle on rows covering every row
# block); the second fills one tile, so K is split in two equal ranges; the
# third is smaller still and normalizes.
CALLS = [("skip", 300, 128, 1800, 12288, synth.NORM_RMSNORM, synth.F16),
         ("big", 100, 264, 520, 136, synth.NORM_NONE, synth.F16),
         ("small", 40, 136, 200, 72, synth.NORM_LAYERNORM, synth.BF16)]


def test_noalloc_equals_fused_ffn_on_two_calls():
    import norm_gemm_amd as ng
    for name, M, K, F, N, norm, dtype in CALLS:
        print(f"noalloc {name}: M={M} K={K} F={F} N={N} norm={norm} dtype={dtype}", flush=True)
        case = synth.make_ffn(f"noalloc_{name}", M, K, F, N, dtype=dtype, norm=norm,
                              gamma=norm != synth.NORM_NONE, beta=norm != synth.NORM_NONE,
                              b1=True, b2=True, seed=M + F)
        A = case.arrays
        u = lambda k: upload(A.get(k), dtype)
        args = (u("x"), u("W1"), u("W2"), u("gamma"), u("beta"), u("b1"), u("b2"))
        ws = torch.empty(ng.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
        y_ref = ng.fused_ffn(*args, eps=1e-5, norm=norm, act="silu", workspace=ws)
        y = ng.fused_ffn_noalloc(*args, eps=1e-5, norm=norm, act="silu")
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), name
        if M * N * F > 10 ** 9:
            rows = tile_indices(M, 128, seed=3, interior=1)
            assert_close(to_f64(y)[rows], oracle.run_case(case, rows=rows), what=f"noalloc {name}")
        else:
            assert_close(to_f64(y), oracle.run_case(case), what=f"noalloc {name}")


def test_noalloc_rejects_requests_beyond_its_scratch():
    import norm_gemm_amd as ng
    M, K, F, N = 512, 64, 65536 + 128, 64          # h = 64 MiB + 128 KiB
    x = torch.zeros(M, K, dtype=torch.float16, device="cuda")
    w1 = torch.zeros(F, K, dtype=torch.float16, device="cuda")
    w2 = torch.zeros(N, F, dtype=torch.float16, device="cuda")
    with pytest.raises(ng.NormGemmError) as e:
        ng.fused_ffn_noalloc(x, w1, w2)
    assert e.value.status == -10
