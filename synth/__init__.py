"""Seeded synthetic inputs for the normalization-prologue GEMM workloads.

This module only draws random numbers and rounds them to the 16-bit storage
formats; it holds none of the method's arithmetic (no normalization, no
products, no activation). Both the CPU oracle and the GPU path consume the bit
patterns produced here, so the two sides see identical inputs.

Recipe (stated once here and in the design notes):

* Generator: ``numpy.random.Generator(PCG64(seed))``; draws are float32
  standard normals, scaled to N(mean, variance) in float32, then rounded to
  the storage dtype with round-to-nearest-even (fp16 via numpy's own cast,
  bf16 via :func:`f32_to_bf16_bits`).
* ``N(a, b)`` is read as mean ``a`` and *variance* ``b``: weights use the
  fan-in variance ``1/K``, so their std is ``K**-0.5``.
* Draw order per case: x, gamma, beta, W (or W1, W2), bias (or b1, b2); for
  the post-GEMM normalization, whose gamma / beta act on the output row: x, W,
  bias, gamma, beta. Tensors a case does not have are not drawn.
* Large tensors are drawn in fixed-size chunks from the same stream, which
  yields the same values as one draw of the whole tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

F16 = 0
BF16 = 1
NORM_NONE, NORM_LAYERNORM, NORM_RMSNORM = 0, 1, 2
ACT_NONE, ACT_SILU, ACT_RELU, ACT_GELU = 0, 1, 2, 3

_CHUNK = 1 << 24  # elements per draw; fixed so that results never depend on it


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (RNE) and return the raw bits."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return the raw bits.

    bfloat16 is the upper half of a binary32 word; rounding to nearest-even
    adds 0x7FFF plus the lowest kept bit before truncating. NaNs keep a quiet
    NaN payload.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return rounded


def bits_from_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_f16_bits(a) if dtype == F16 else f32_to_bf16_bits(a)


def normal_bits(rng: np.random.Generator, shape, mean: float, var: float,
                dtype: int) -> np.ndarray:
    """Draw ``prod(shape)`` i.i.d. N(mean, var) values, rounded to ``dtype``."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    std = np.float32(math.sqrt(var))
    mu = np.float32(mean)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        z = rng.standard_normal(e - s, dtype=np.float32)
        z *= std
        z += mu
        out[s:e] = bits_from_f32(z, dtype)
    return out.reshape(shape)


@dataclass
class Case:
    """One workload: shapes, options and the input bit patterns (uint16)."""
    name: str
    kind: str                      # "norm_gemm", "ffn", "gated_ffn" or "gemm_norm"
    dtype: int
    M: int
    K: int
    N: int
    F: int = 0                     # FFN hidden width (kind == "ffn")
    norm: int = NORM_NONE
    act: int = ACT_NONE
    eps: float = 1e-5
    arrays: Dict[str, Optional[np.ndarray]] = field(default_factory=dict)

    def get(self, key: str) -> Optional[np.ndarray]:
        return self.arrays.get(key)


def make_norm_gemm(name: str, M: int, K: int, N: int, *, dtype: int = F16,
                   norm: int = NORM_LAYERNORM, act: int = ACT_NONE,
                   eps: float = 1e-5, gamma: bool = True, beta: bool = True,
                   bias: bool = True, seed: int = 0, x_mean: float = 0.0,
                   x_var: float = 1.0) -> Case:
    """x[M,K] ~ N(x_mean, x_var), gamma ~ N(1, 0.1), beta ~ N(0, 0.1),
    W[N,K] ~ N(0, 1/K), bias[N] ~ N(0, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    arr: Dict[str, Optional[np.ndarray]] = {}
    arr["x"] = normal_bits(rng, (M, K), x_mean, x_var, dtype)
    arr["gamma"] = normal_bits(rng, (K,), 1.0, 0.1, dtype) if gamma else None
    arr["beta"] = normal_bits(rng, (K,), 0.0, 0.1, dtype) if beta else None
    arr["W"] = normal_bits(rng, (N, K), 0.0, 1.0 / K, dtype)
    arr["bias"] = normal_bits(rng, (N,), 0.0, 0.1, dtype) if bias else None
    return Case(name, "norm_gemm", dtype, M, K, N, 0, norm, act, eps, arr)


def make_ffn(name: str, M: int, K: int, F: int, N: int, *, dtype: int = F16,
             norm: int = NORM_NONE, act: int = ACT_SILU, eps: float = 1e-5,
             gamma: bool = False, beta: bool = False, b1: bool = False,
             b2: bool = False, seed: int = 0) -> Case:
    """x[M,K] ~ N(0,1), W1[F,K] ~ N(0, 1/K), W2[N,F] ~ N(0, 1/F); optional
    gamma/beta as in :func:`make_norm_gemm`, b1/b2 ~ N(0, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    arr: Dict[str, Optional[np.ndarray]] = {}
    arr["x"] = normal_bits(rng, (M, K), 0.0, 1.0, dtype)
    arr["gamma"] = normal_bits(rng, (K,), 1.0, 0.1, dtype) if gamma else None
    arr["beta"] = normal_bits(rng, (K,), 0.0, 0.1, dtype) if beta else None
    arr["W1"] = normal_bits(rng, (F, K), 0.0, 1.0 / K, dtype)
    arr["W2"] = normal_bits(rng, (N, F), 0.0, 1.0 / F, dtype)
    arr["b1"] = normal_bits(rng, (F,), 0.0, 0.1, dtype) if b1 else None
    arr["b2"] = normal_bits(rng, (N,), 0.0, 0.1, dtype) if b2 else None
    return Case(name, "ffn", dtype, M, K, N, F, norm, act, eps, arr)


def make_gated_ffn(name: str, M: int, K: int, F: int, N: int, *, dtype: int = F16,
                   norm: int = NORM_NONE, act: int = ACT_SILU, eps: float = 1e-5,
                   gamma: bool = False, beta: bool = False, b1: bool = False,
                   b2: bool = False, seed: int = 0) -> Case:
    """Gated FFN: x[M,K] ~ N(0,1), W1 = [W_gate; W_up] [2F,K] ~ N(0, 1/K),
    W2[N,F] ~ N(0, 1/F); optional gamma/beta, b1 [2F] and b2 ~ N(0, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    arr: Dict[str, Optional[np.ndarray]] = {}
    arr["x"] = normal_bits(rng, (M, K), 0.0, 1.0, dtype)
    arr["gamma"] = normal_bits(rng, (K,), 1.0, 0.1, dtype) if gamma else None
    arr["beta"] = normal_bits(rng, (K,), 0.0, 0.1, dtype) if beta else None
    arr["W1"] = normal_bits(rng, (2 * F, K), 0.0, 1.0 / K, dtype)
    arr["W2"] = normal_bits(rng, (N, F), 0.0, 1.0 / F, dtype)
    arr["b1"] = normal_bits(rng, (2 * F,), 0.0, 0.1, dtype) if b1 else None
    arr["b2"] = normal_bits(rng, (N,), 0.0, 0.1, dtype) if b2 else None
    return Case(name, "gated_ffn", dtype, M, K, N, F, norm, act, eps, arr)


def make_gemm_norm(name: str, M: int, K: int, N: int, *, dtype: int = F16,
                   norm: int = NORM_RMSNORM, eps: float = 1e-5, bias: bool = False,
                   gamma: bool = True, beta: bool = False, seed: int = 0) -> Case:
    """Post-GEMM normalization: x[M,K] ~ N(0,1), W[N,K] ~ N(0, 1/K), then the
    output row's bias[N] ~ N(0, 0.1), gamma[N] ~ N(1, 0.1), beta[N] ~ N(0, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    arr: Dict[str, Optional[np.ndarray]] = {}
    arr["x"] = normal_bits(rng, (M, K), 0.0, 1.0, dtype)
    arr["W"] = normal_bits(rng, (N, K), 0.0, 1.0 / K, dtype)
    arr["bias"] = normal_bits(rng, (N,), 0.0, 0.1, dtype) if bias else None
    arr["gamma"] = normal_bits(rng, (N,), 1.0, 0.1, dtype) if gamma else None
    arr["beta"] = normal_bits(rng, (N,), 0.0, 0.1, dtype) if beta else None
    return Case(name, "gemm_norm", dtype, M, K, N, 0, norm, ACT_NONE, eps, arr)


# The five workloads of the hot path, by what they are.
def ln_linear_bias_64x256(seed: int = 0) -> Case:
    return make_norm_gemm("ln_linear_bias_x64x256_w256x256_f16", 64, 256, 256,
                          norm=NORM_LAYERNORM, eps=1e-5, seed=seed)


def ln_linear_bias_1024x8192(seed: int = 0) -> Case:
    return make_norm_gemm("ln_linear_bias_x1024x8192_w8192x8192_f16", 1024, 8192,
                          8192, norm=NORM_LAYERNORM, eps=1e-5, seed=seed)


def rms_matmul_silu_512x14336(seed: int = 0) -> Case:
    return make_norm_gemm("rms_matmul_silu_x512x14336_w49152x14336_f16", 512,
                          14336, 49152, norm=NORM_RMSNORM, act=ACT_SILU,
                          eps=1e-6, beta=False, bias=False, seed=seed)


def ffn_silu_512x14336x49152(seed: int = 0) -> Case:
    return make_ffn("ffn_silu_x512x14336_w1_49152_w2_14336_f16", 512, 14336,
                    49152, 14336, act=ACT_SILU, seed=seed)


def gated_ffn_swiglu_512x8192x28672(seed: int = 0) -> Case:
    """RMSNorm -> [gate; up] -> SiLU(gate) * up -> down, LLaMA-2-70B FFN sizes."""
    return make_gated_ffn("gated_ffn_swiglu_rms_x512x8192_w1_57344_w2_8192_f16", 512, 8192,
                          28672, 8192, norm=NORM_RMSNORM, act=ACT_SILU, eps=1e-5, gamma=True,
                          seed=seed)


def attn_out_rmsnorm_512x8192(seed: int = 0) -> Case:
    """The attention output projection with the RMSNorm after it (LLaMA-2-70B
    hidden size 8192, 512 tokens): x[512, 8192] . W[8192, 8192]^T, then
    RMSNorm with gamma over the 8192 outputs, fp16."""
    return make_gemm_norm("attn_out_rmsnorm_x512x8192_w8192x8192_f16", 512, 8192, 8192,
                          norm=NORM_RMSNORM, eps=1e-5, gamma=True, seed=seed)


def decode_rms_gemm_8192x28672(M: int, seed: int = 0) -> Case:
    return make_norm_gemm(f"decode_rms_gemm_m{M}_x{M}x8192_w28672x8192_bf16", M,
                          8192, 28672, dtype=BF16, norm=NORM_RMSNORM,
                          eps=1e-6, beta=False, bias=False, seed=seed)


WORKLOADS = {
    "ln_linear_bias_64x256": ln_linear_bias_64x256,
    "ln_linear_bias_1024x8192": ln_linear_bias_1024x8192,
    "rms_matmul_silu_512x14336": rms_matmul_silu_512x14336,
    "ffn_silu_512x14336x49152": ffn_silu_512x14336x49152,
    "gated_ffn_swiglu_512x8192x28672": gated_ffn_swiglu_512x8192x28672,
    "attn_out_rmsnorm_512x8192": attn_out_rmsnorm_512x8192,
    "decode_rms_gemm_m1": lambda seed=0: decode_rms_gemm_8192x28672(1, seed),
    "decode_rms_gemm_m8": lambda seed=0: decode_rms_gemm_8192x28672(8, seed),
    "decode_rms_gemm_m32": lambda seed=0: decode_rms_gemm_8192x28672(32, seed),
}
