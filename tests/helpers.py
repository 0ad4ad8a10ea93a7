"""Shared helpers of the GPU tests: upload seeded inputs, call the library,
compare with the oracle under the acceptance metric."""
from __future__ import annotations

import numpy as np
import torch

import synth

TOL = 1e-2  # max |gpu - ref| / (|ref| + 1), fp16/bf16 output, fp32 accumulation


def tdtype(dtype: int):
    return torch.float16 if dtype == synth.F16 else torch.bfloat16


def upload(bits, dtype: int, device="cuda"):
    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(tdtype(dtype)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    assert gpu.shape == ref.shape
    if gpu.size == 0:
        return 0.0
    return float(np.max(np.abs(gpu - ref) / (np.abs(ref) + 1.0)))


def assert_close(gpu: np.ndarray, ref: np.ndarray, tol: float = TOL, what: str = ""):
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(gpu[fin])), f"{what}: non-finite GPU value where ref is finite"
    err = rel_err(gpu[fin], ref[fin])
    assert err <= tol, f"{what}: max |gpu-ref|/(|ref|+1) = {err:.3e} > {tol}"
    return err


def run_case_gpu(case, device="cuda"):
    """Run a synth.Case through the library; returns the output tensor."""
    import norm_gemm_amd as ng
    A = case.arrays
    up = lambda k: upload(A.get(k), case.dtype, device)
    norm = case.norm
    act = case.act
    if case.kind == "gated_ffn":
        return ng.fused_gated_ffn(up("x"), up("W1"), up("W2"), up("gamma"), up("beta"), up("b1"),
                                  up("b2"), eps=case.eps, norm=norm, act=act)
    if case.kind == "gemm_norm":
        return ng.fused_gemm_norm(up("x"), up("W"), up("bias"), up("gamma"), up("beta"),
                                  eps=case.eps, norm=norm)
    if case.kind == "ffn":
        return ng.fused_ffn(up("x"), up("W1"), up("W2"), up("gamma"), up("beta"), up("b1"),
                            up("b2"), eps=case.eps, norm=norm, act=act)
    return ng.fused_norm_gemm(up("x"), up("W"), up("gamma"), up("beta"), up("bias"),
                              eps=case.eps, norm=norm, act=act)


def tile_indices(n: int, tile: int, seed: int, interior: int = 1):
    """Both edges of every `tile`-sized block of range(n) plus `interior`
    seeded indices inside each block: every tile of the output is compared,
    with its first and last row (or column) among them."""
    rng = np.random.default_rng(seed)
    out = set()
    for b0 in range(0, n, tile):
        b1 = min(n, b0 + tile) - 1
        out.update((b0, b1))
        if b1 > b0 + 1 and interior:
            out.update(int(v) for v in rng.integers(b0 + 1, b1, size=interior))
    return sorted(out)


def one_ulp(dtype) -> float:
    """Bound of |a - b| / (|b| + 1) for two outputs that differ only in the
    fp32 summation order of the same products (a split K against an unsplit
    one): each is rounded once to the output type, so they may differ by one
    unit in the last place, 2^-10 |y| in fp16 and 2^-7 |y| in bf16 (plus a
    margin for the fp32 sums themselves)."""
    import synth
    return (2.0 ** -10 if dtype == synth.F16 else 2.0 ** -7) + 1e-4
