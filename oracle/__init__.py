"""ctypes wrapper of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. Product code never
imports this package, and the GPU path shares no code with it.

Inputs are numpy ``uint16`` arrays holding fp16/bf16 bit patterns (as made
by :mod:`synth`); outputs are float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at a deliberately mutated build of oracle.c to
# show that the pins catch the mutation; nothing else sets this.
_LIB_OVERRIDE = os.environ.get("NORM_GEMM_ORACLE_LIB")

F16, BF16 = 0, 1
NORM_NONE, NORM_LAYERNORM, NORM_RMSNORM = 0, 1, 2
ACT_NONE, ACT_SILU, ACT_RELU, ACT_GELU = 0, 1, 2, 3


# gcc flags of the oracle library: portable x86-64 code (it is built on one
# host and may run on another), OpenMP over output elements.
COMPILE_FLAGS = ("-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp")


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (portable x86-64 code, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", *COMPILE_FLAGS, "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(path)
        p16 = ctypes.POINTER(ctypes.c_uint16)
        pi64 = ctypes.POINTER(ctypes.c_int64)
        pf64 = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_normalize.argtypes = [p16, p16, p16, i64, i64, ctypes.c_float,
                                       ctypes.c_int, ctypes.c_int, pi64, i64, pf64]
        L.oracle_normalize.restype = ctypes.c_int
        L.oracle_norm_gemm.argtypes = [p16, p16, p16, p16, p16, i64, i64, i64,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, pi64, i64, pi64, i64, pf64]
        L.oracle_norm_gemm.restype = ctypes.c_int
        L.oracle_ffn.argtypes = [p16, p16, p16, p16, p16, p16, p16, i64, i64, i64,
                                 i64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, pi64, i64, pi64, i64, pf64]
        L.oracle_ffn.restype = ctypes.c_int
        L.oracle_gated_ffn.argtypes = L.oracle_ffn.argtypes
        L.oracle_gated_ffn.restype = ctypes.c_int
        L.oracle_fold_weights.argtypes = [p16, p16, p16, p16, i64, i64, ctypes.c_int, pf64,
                                          pf64, pf64]
        L.oracle_fold_weights.restype = ctypes.c_int
        L.oracle_norm_gemm_folded.argtypes = [p16, pf64, pf64, pf64, i64, i64, i64,
                                              ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, pi64, i64, pi64, i64, pf64]
        L.oracle_norm_gemm_folded.restype = ctypes.c_int
        L.oracle_gemm_norm.argtypes = [p16, p16, p16, p16, p16, i64, i64, i64, ctypes.c_float,
                                       ctypes.c_int, ctypes.c_int, pi64, i64, pi64, i64, pf64]
        L.oracle_gemm_norm.restype = ctypes.c_int
        _lib = L
    return _lib


def _u16(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _idx(ix: Optional[Sequence[int]], n: int):
    arr = np.arange(n, dtype=np.int64) if ix is None else np.ascontiguousarray(ix, dtype=np.int64)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(int(bits))


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Decode an array of 16-bit patterns with the oracle's own decoder."""
    f = lib().oracle_bf16_to_f64 if dtype == BF16 else lib().oracle_f16_to_f64
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    table = np.array([f(i) for i in range(65536)], dtype=np.float64)
    return table[flat].reshape(np.shape(bits))


def normalize(x, gamma, beta, eps: float, norm: int, dtype: int,
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    M, K = x.shape
    x, px = _u16(x)
    g, pg = _u16(gamma)
    b, pb = _u16(beta)
    r, pr = _idx(rows, M)
    out = np.empty((len(r), K), dtype=np.float64)
    rc = lib().oracle_normalize(px, pg, pb, M, K, eps, norm, dtype, pr, len(r),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_normalize failed ({rc})")
    return out


def norm_gemm(x, gamma, beta, W, bias, eps: float, norm: int, act: int, dtype: int,
              rows: Optional[Sequence[int]] = None,
              cols: Optional[Sequence[int]] = None) -> np.ndarray:
    M, K = x.shape
    N = W.shape[0]
    assert W.shape[1] == K
    x, px = _u16(x)
    g, pg = _u16(gamma)
    b, pb = _u16(beta)
    w, pw = _u16(W)
    bi, pbi = _u16(bias)
    r, pr = _idx(rows, M)
    c, pc = _idx(cols, N)
    out = np.empty((len(r), len(c)), dtype=np.float64)
    rc = lib().oracle_norm_gemm(px, pg, pb, pw, pbi, M, N, K, eps, norm, act, dtype,
                                pr, len(r), pc, len(c),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_norm_gemm failed ({rc})")
    return out


def ffn(x, gamma, beta, W1, b1, W2, b2, eps: float, norm: int, act: int, dtype: int,
        rows: Optional[Sequence[int]] = None,
        cols: Optional[Sequence[int]] = None, gated: bool = False) -> np.ndarray:
    """y = act(a W1^T + b1) W2^T + b2; gated: W1 = [W_gate; W_up] is [2F, K] and
    h = act(a W_gate^T + b_gate) * (a W_up^T + b_up)."""
    M, K = x.shape
    F = W1.shape[0] // 2 if gated else W1.shape[0]
    N = W2.shape[0]
    assert W1.shape[1] == K and W2.shape[1] == F and (not gated or W1.shape[0] == 2 * F)
    x, px = _u16(x)
    g, pg = _u16(gamma)
    b, pb = _u16(beta)
    w1, pw1 = _u16(W1)
    bb1, pb1 = _u16(b1)
    w2, pw2 = _u16(W2)
    bb2, pb2 = _u16(b2)
    r, pr = _idx(rows, M)
    c, pc = _idx(cols, N)
    out = np.empty((len(r), len(c)), dtype=np.float64)
    fn = lib().oracle_gated_ffn if gated else lib().oracle_ffn
    rc = fn(px, pg, pb, pw1, pb1, pw2, pb2, M, K, F, N, eps, norm, act,
            dtype, pr, len(r), pc, len(c),
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_ffn failed ({rc})")
    return out


def run_case(case, rows=None, cols=None) -> np.ndarray:
    """Oracle output for a :class:`synth.Case` (optionally a row/col sample)."""
    A = case.arrays
    if case.kind == "gemm_norm":
        return gemm_norm(A["x"], A["W"], A.get("bias"), A.get("gamma"), A.get("beta"),
                         case.eps, case.norm, case.dtype, rows, cols)
    if case.kind in ("ffn", "gated_ffn"):
        return ffn(A["x"], A.get("gamma"), A.get("beta"), A["W1"], A.get("b1"),
                   A["W2"], A.get("b2"), case.eps, case.norm, case.act, case.dtype,
                   rows, cols, gated=case.kind == "gated_ffn")
    return norm_gemm(A["x"], A.get("gamma"), A.get("beta"), A["W"], A.get("bias"),
                     case.eps, case.norm, case.act, case.dtype, rows, cols)


def _f64(a: Optional[np.ndarray]):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fold_weights(W, gamma, beta, bias, dtype: int, want_w: bool = True):
    """Folded weights of the inference-mode strategy: (W' = W * gamma [N,K]
    fp64 or None, c1 = W' 1 [N], c2 = W beta + bias [N])."""
    N, K = W.shape
    w, pw = _u16(W)
    g, pg = _u16(gamma)
    b, pb = _u16(beta)
    bi, pbi = _u16(bias)
    Wf = np.empty((N, K), dtype=np.float64) if want_w else None
    c1 = np.empty(N, dtype=np.float64)
    c2 = np.empty(N, dtype=np.float64)
    pf = None if Wf is None else Wf.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = lib().oracle_fold_weights(pw, pg, pb, pbi, N, K, dtype, pf,
                                   c1.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                   c2.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_fold_weights failed ({rc})")
    return Wf, c1, c2


def norm_gemm_folded(x, Wf, c1, c2, eps: float, norm: int, act: int, dtype: int,
                     rows: Optional[Sequence[int]] = None,
                     cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """y = act(r (x Wf^T - mu c1) + c2) with the definition's row statistics."""
    M, K = x.shape
    N = Wf.shape[0]
    assert Wf.shape[1] == K and c1.shape == (N,) and c2.shape == (N,)
    x, px = _u16(x)
    wf, pwf = _f64(Wf)
    a1, p1 = _f64(c1)
    a2, p2 = _f64(c2)
    r, pr = _idx(rows, M)
    c, pc = _idx(cols, N)
    out = np.empty((len(r), len(c)), dtype=np.float64)
    rc = lib().oracle_norm_gemm_folded(px, pwf, p1, p2, M, N, K, eps, norm, act, dtype,
                                       pr, len(r), pc, len(c),
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_norm_gemm_folded failed ({rc})")
    return out


def gemm_norm(x, W, bias, gamma, beta, eps: float, norm: int, dtype: int,
              rows: Optional[Sequence[int]] = None,
              cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """y = norm_affine(x W^T + bias) over each output row (gamma, beta [N])."""
    M, K = x.shape
    N = W.shape[0]
    assert W.shape[1] == K
    x, px = _u16(x)
    w, pw = _u16(W)
    bi, pbi = _u16(bias)
    g, pg = _u16(gamma)
    b, pb = _u16(beta)
    r, pr = _idx(rows, M)
    c, pc = _idx(cols, N)
    out = np.empty((len(r), len(c)), dtype=np.float64)
    rc = lib().oracle_gemm_norm(px, pw, pbi, pg, pb, M, N, K, eps, norm, dtype, pr, len(r),
                                pc, len(c), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError(f"oracle_gemm_norm failed ({rc})")
    return out
