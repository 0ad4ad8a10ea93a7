"""Seeded sweep of random shapes through every entry point, each output
compared with the fp64 oracle in full.

The shapes are drawn once from a fixed seed, so the sweep is the same on
every run: M from 1 to 700 (the skinny kernels up to 32 rows, the tiled ones
above), K with and without K % 8 == 0, operands with and without 16-byte
alignment (a one-element offset into a larger buffer), every normalization,
activation and dtype, gamma / beta / bias present or not; FFN and gated FFN
chains; post-GEMM normalization on aligned shapes. A routing or tail bug
that only some shapes reach shows up here with the case that found it."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, assert_close, to_f64

pytestmark = pytest.mark.gpu

NORMS = ("none", "layernorm", "rmsnorm")
ACTS = ("none", "silu", "relu", "gelu")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import norm_gemm_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def place(a, dtype, misalign):
    """Device tensor with the bits of `a`, 16-byte aligned or one element off."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")
    if not misalign:
        return t.view(torch.float16 if dtype == synth.F16 else torch.bfloat16)
    buf = torch.empty(t.numel() + 8, dtype=torch.int16, device="cuda")
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    return v.view(torch.float16 if dtype == synth.F16 else torch.bfloat16)


def _gemm_cases():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(60):
        M = int(rng.integers(1, 33)) if i % 3 == 0 else int(rng.integers(33, 701))
        aligned = i % 4 != 3
        K = int(rng.integers(8, 1201))
        if aligned:
            K = max(8, K - K % 8)
        N = int(rng.integers(1, 2101))
        norm = int(rng.integers(0, 3))
        act = int(rng.integers(0, 4))
        dtype = synth.F16 if rng.integers(0, 2) == 0 else synth.BF16
        gamma, beta, bias = (bool(rng.integers(0, 2)) for _ in range(3))
        out.append((i, M, K, N, norm, act, dtype, gamma and norm > 0, beta and norm > 0, bias,
                    not aligned))
    return out


@pytest.mark.parametrize("i,M,K,N,norm,act,dtype,gamma,beta,bias,misalign", _gemm_cases(),
                         ids=lambda v: str(v))
def test_random_norm_gemm(i, M, K, N, norm, act, dtype, gamma, beta, bias, misalign):
    import norm_gemm_amd as ng
    eps = 1e-5 if norm == synth.NORM_LAYERNORM else 1e-6
    case = synth.make_norm_gemm(f"rand_{i}", M, K, N, dtype=dtype, norm=norm, act=act, eps=eps,
                                gamma=gamma, beta=beta, bias=bias, seed=1000 + i)
    A = case.arrays
    p = lambda k: place(A.get(k), dtype, misalign)
    print(f"case {i}: M={M} K={K} N={N} norm={norm} act={act} dtype={dtype} "
          f"gamma={gamma} beta={beta} bias={bias} misalign={misalign}", flush=True)
    y = ng.fused_norm_gemm(p("x"), p("W"), p("gamma"), p("beta"), p("bias"), eps=eps,
                           norm=NORMS[norm], act=ACTS[act])
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)


def _ffn_cases():
    rng = np.random.default_rng(7)
    out = []
    for i in range(16):
        M = int(rng.integers(1, 33)) if i % 4 == 0 else int(rng.integers(33, 400))
        K = int(rng.integers(1, 64)) * 8
        F = int(rng.integers(8, 900))
        N = int(rng.integers(1, 600))
        norm = int(rng.integers(0, 3))
        act = int(rng.integers(1, 4))
        dtype = synth.F16 if i % 2 == 0 else synth.BF16
        out.append((i, M, K, F, N, norm, act, dtype, i % 3 == 1))
    return out


@pytest.mark.parametrize("i,M,K,F,N,norm,act,dtype,gated", _ffn_cases(), ids=lambda v: str(v))
def test_random_ffn(i, M, K, F, N, norm, act, dtype, gated):
    import norm_gemm_amd as ng
    make = synth.make_gated_ffn if gated else synth.make_ffn
    case = make(f"rand_ffn_{i}", M, K, F, N, dtype=dtype, norm=norm, act=act, eps=1e-5,
                gamma=norm > 0, beta=norm == synth.NORM_LAYERNORM, b1=True, b2=i % 2 == 0,
                seed=2000 + i)
    A = case.arrays
    p = lambda k: place(A.get(k), dtype, False)
    print(f"ffn case {i}: M={M} K={K} F={F} N={N} norm={norm} act={act} dtype={dtype} "
          f"gated={gated}", flush=True)
    call = ng.fused_gated_ffn if gated else ng.fused_ffn
    y = call(p("x"), p("W1"), p("W2"), p("gamma"), p("beta"), p("b1"), p("b2"), eps=1e-5,
             norm=NORMS[norm], act=ACTS[act])
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)


def _gemm_norm_cases():
    rng = np.random.default_rng(11)
    out = []
    for i in range(12):
        M = int(rng.integers(1, 400))
        K = int(rng.integers(1, 150)) * 8
        N = int(rng.integers(1, 3000))
        norm = 1 + int(rng.integers(0, 2))
        dtype = synth.F16 if i % 2 == 0 else synth.BF16
        out.append((i, M, K, N, norm, dtype, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,M,K,N,norm,dtype,bias,beta", _gemm_norm_cases(), ids=lambda v: str(v))
def test_random_gemm_norm(i, M, K, N, norm, dtype, bias, beta):
    import norm_gemm_amd as ng
    case = synth.make_gemm_norm(f"rand_gn_{i}", M, K, N, dtype=dtype, norm=norm, bias=bias,
                                gamma=True, beta=beta, eps=1e-5, seed=3000 + i)
    A = case.arrays
    p = lambda k: place(A.get(k), dtype, False)
    print(f"gemm_norm case {i}: M={M} K={K} N={N} norm={norm} dtype={dtype}", flush=True)
    y = ng.fused_gemm_norm(p("x"), p("W"), p("bias"), p("gamma"), p("beta"), eps=1e-5,
                           norm=NORMS[norm])
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.run_case(case), TOL, case.name)
