"""Python binding of ``libnormgemm.so``: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; PyTorch
supplies device memory and the stream. The functions mirror the C ABI in
``include/norm_gemm.h`` and keep its names:

* :func:`fused_norm_gemm` -- y = act(norm_affine(x) @ W.T + bias)
* :func:`fused_ffn` -- y = act(norm_affine(x) @ W1.T + b1) @ W2.T + b2
* :func:`fused_ffn_noalloc` -- the FFN with the library's static workspace
* :func:`norm_gemm_fold_weights`, :func:`fused_norm_gemm_folded` --
  inference-mode folding of gamma / beta into the weights
* :func:`fused_gemm_norm` -- y = norm_affine(x @ W.T + bias) over output rows
* :func:`fused_ffn_workspace_size`, :func:`norm_gemm_status_string`,
  :func:`norm_gemm_abi_version`

There is no fallback: importing this package without the built library
raises ImportError, and a failing status raises :class:`NormGemmError`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

# torch first: it loads the HIP runtime that the library then shares (same
# soname), so streams and device pointers from torch are valid in the library.
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libnormgemm.so")

NORMS = {"none": 0, "layernorm": 1, "rmsnorm": 2}
ACTS = {"none": 0, "silu": 1, "relu": 2, "gelu": 3}
DTYPES = {torch.float16: 0, torch.bfloat16: 1}

# Symbols declared in include/norm_gemm.h.
EXPORTED = ("fused_norm_gemm", "fused_ffn", "fused_ffn_workspace_size", "fused_gated_ffn",
            "fused_gated_ffn_workspace_size", "fused_ffn_noalloc", "norm_gemm_fold_weights",
            "fused_norm_gemm_folded", "fused_gemm_norm", "fused_gemm_norm_workspace_size",
            "norm_gemm_status_string", "norm_gemm_abi_version")

# Size of the static device array behind fused_ffn_noalloc
# (NG_FFN_NOALLOC_SCRATCH_BYTES in include/norm_gemm.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


class NormGemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {norm_gemm_status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(f"{LIBRARY_PATH} is not built; run `python norm_gemm_amd/build.py` from the repository root")
    L = ctypes.CDLL(LIBRARY_PATH)
    vp, i64, f32, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    L.fused_norm_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, ci, ci, ci, vp]
    L.fused_norm_gemm.restype = ci
    L.fused_ffn_workspace_size.argtypes = [i64, i64, ci]
    L.fused_ffn_workspace_size.restype = sz
    L.fused_ffn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, ci, ci,
                            ci, vp, sz, vp]
    L.fused_ffn.restype = ci
    L.fused_gated_ffn_workspace_size.argtypes = [i64, i64, ci]
    L.fused_gated_ffn_workspace_size.restype = sz
    L.fused_gated_ffn.argtypes = L.fused_ffn.argtypes
    L.fused_gated_ffn.restype = ci
    L.fused_ffn_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, ci,
                                    ci, ci, vp]
    L.fused_ffn_noalloc.restype = ci
    L.norm_gemm_fold_weights.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, vp]
    L.norm_gemm_fold_weights.restype = ci
    L.fused_norm_gemm_folded.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, f32, ci, ci, ci, vp]
    L.fused_norm_gemm_folded.restype = ci
    L.fused_gemm_norm_workspace_size.argtypes = [i64, i64]
    L.fused_gemm_norm_workspace_size.restype = sz
    L.fused_gemm_norm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, ci, ci, vp, sz, vp]
    L.fused_gemm_norm.restype = ci
    L.norm_gemm_status_string.argtypes = [ci]
    L.norm_gemm_status_string.restype = ctypes.c_char_p
    L.norm_gemm_abi_version.argtypes = []
    L.norm_gemm_abi_version.restype = ci
    return L


lib = _load()


def norm_gemm_status_string(status: int) -> str:
    return lib.norm_gemm_status_string(int(status)).decode()


def norm_gemm_abi_version() -> int:
    return int(lib.norm_gemm_abi_version())


def fused_ffn_workspace_size(M: int, F: int, dtype) -> int:
    d = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.fused_ffn_workspace_size(int(M), int(F), d))


def fused_gated_ffn_workspace_size(M: int, F: int, dtype) -> int:
    d = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.fused_gated_ffn_workspace_size(int(M), int(F), d))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, dtype, device, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _enum(table, value, name):
    if isinstance(value, str):
        if value not in table:
            raise ValueError(f"unknown {name} {value!r}; choose from {sorted(table)}")
        return table[value]
    return int(value)


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fused_norm_gemm(x: torch.Tensor, weight: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                    beta: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None, *,
                    eps: float = 1e-5, norm="layernorm", act="none",
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[..., N] = act(norm_affine(x)[..., K] @ weight[N, K].T + bias[N]).

    ``x`` may have leading dimensions (e.g. [batch, seq, hidden]); they are
    flattened into M. Returns ``out`` (allocated when not given).
    """
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError("x must be a tensor with at least one dimension")
    if x.dtype not in DTYPES:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    dev = x.device
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if weight is None or weight.dim() != 2 or weight.shape[1] != K:
        raise ValueError(f"weight must be [N, {K}]")
    N = weight.shape[0]
    _check(x, "x", x.dtype, dev)
    _check(weight, "weight", x.dtype, dev)
    _check(gamma, "gamma", x.dtype, dev, (K,))
    _check(beta, "beta", x.dtype, dev, (K,))
    _check(bias, "bias", x.dtype, dev, (N,))
    lead = tuple(x.shape[:-1])
    if out is None:
        out = torch.empty(lead + (N,), dtype=x.dtype, device=dev)
    _check(out, "out", x.dtype, dev, lead + (N,))
    with torch.cuda.device(dev):
        st = lib.fused_norm_gemm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(weight), _ptr(bias),
                                 _ptr(out), M, N, K, float(eps), _enum(NORMS, norm, "norm"),
                                 _enum(ACTS, act, "act"), DTYPES[x.dtype], _stream(dev, stream))
    if st != 0:
        raise NormGemmError(st, "fused_norm_gemm")
    return out


def fused_ffn(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
              gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
              b1: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None, *,
              eps: float = 1e-5, norm="none", act="silu",
              workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """y = act(norm_affine(x) @ w1[F, K].T + b1) @ w2[N, F].T + b2.

    The intermediate h[M, F] lives in ``workspace`` (a uint8 device tensor of
    at least :func:`fused_ffn_workspace_size` bytes). 8 M N bytes more also
    hold two fp32 partial sums of y, which lets the second GEMM split K when
    its tiles leave CUs idle; the workspace allocated when none is given has
    that room.
    """
    return _ffn(False, x, w1, w2, gamma, beta, b1, b2, eps, norm, act, workspace, out, stream)


def fused_gated_ffn(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
                    gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                    b1: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None, *,
                    eps: float = 1e-5, norm="none", act="silu",
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Gated FFN (SwiGLU with act="silu"): with w1 = [w_gate; w_up] of shape
    [2F, K] (and b1 = [b_gate; b_up] of shape [2F]),
    y = (act(a @ w_gate.T + b_gate) * (a @ w_up.T + b_up)) @ w2[N, F].T + b2,
    a = norm_affine(x). The workspace holds at least
    :func:`fused_gated_ffn_workspace_size` bytes (allocated when not given).
    """
    return _ffn(True, x, w1, w2, gamma, beta, b1, b2, eps, norm, act, workspace, out, stream)


def fused_ffn_noalloc(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
                      gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                      b1: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None, *,
                      eps: float = 1e-5, norm="none", act="silu",
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """:func:`fused_ffn` whose intermediate lives in the library's static
    per-device array (:data:`NOALLOC_SCRATCH_BYTES`): the library call
    allocates nothing. Pass ``out`` to keep this function free of
    allocations too. Calls that overlap in time on one device race."""
    return _ffn(False, x, w1, w2, gamma, beta, b1, b2, eps, norm, act, None, out, stream,
                noalloc=True)


def _ffn(gated, x, w1, w2, gamma, beta, b1, b2, eps, norm, act, workspace, out, stream,
         noalloc=False):
    what = "fused_gated_ffn" if gated else ("fused_ffn_noalloc" if noalloc else "fused_ffn")
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError("x must be a tensor with at least one dimension")
    if x.dtype not in DTYPES:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    dev = x.device
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if w1 is None or w1.dim() != 2 or w1.shape[1] != K or (gated and w1.shape[0] % 2):
        raise ValueError(f"w1 must be [{'2F' if gated else 'F'}, {K}]")
    F = w1.shape[0] // 2 if gated else w1.shape[0]
    if w2 is None or w2.dim() != 2 or w2.shape[1] != F:
        raise ValueError(f"w2 must be [N, {F}]")
    N = w2.shape[0]
    for t, name, shp in ((x, "x", None), (w1, "w1", None), (w2, "w2", None), (gamma, "gamma", (K,)),
                         (beta, "beta", (K,)), (b1, "b1", (w1.shape[0],)), (b2, "b2", (N,))):
        _check(t, name, x.dtype, dev, shp)
    if not noalloc:
        need = (fused_gated_ffn_workspace_size if gated else fused_ffn_workspace_size)(M, F, x.dtype)
        if workspace is None:
            # plain FFN: room for the two fp32 partial sums of y past h (the
            # gated FFN's [gate | up] area already holds them when F >= 2 N)
            workspace = torch.empty(need + (0 if gated else 8 * M * N), dtype=torch.uint8,
                                    device=dev)
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on x's device")
    lead = tuple(x.shape[:-1])
    if out is None:
        out = torch.empty(lead + (N,), dtype=x.dtype, device=dev)
    _check(out, "out", x.dtype, dev, lead + (N,))
    with torch.cuda.device(dev):
        common = (_ptr(x), _ptr(gamma), _ptr(beta), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                  _ptr(out), M, K, F, N, float(eps), _enum(NORMS, norm, "norm"),
                  _enum(ACTS, act, "act"), DTYPES[x.dtype])
        if noalloc:
            st = lib.fused_ffn_noalloc(*common, _stream(dev, stream))
        else:
            fn = lib.fused_gated_ffn if gated else lib.fused_ffn
            ws_bytes = workspace.numel() * workspace.element_size()
            st = fn(*common, _ptr(workspace), ws_bytes, _stream(dev, stream))
    if st != 0:
        raise NormGemmError(st, what)
    return out


def norm_gemm_fold_weights(weight: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                           beta: Optional[torch.Tensor] = None,
                           bias: Optional[torch.Tensor] = None, *, stream=None):
    """Folded weights for :func:`fused_norm_gemm_folded`: returns (w_folded
    [N, K] = weight * gamma rounded once, c1 = w_folded.sum(1) in fp32,
    c2 = weight @ beta + bias in fp32)."""
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a [N, K] tensor")
    if weight.dtype not in DTYPES:
        raise ValueError(f"weight must be float16 or bfloat16, got {weight.dtype}")
    dev = weight.device
    N, K = weight.shape
    _check(weight, "weight", weight.dtype, dev)
    _check(gamma, "gamma", weight.dtype, dev, (K,))
    _check(beta, "beta", weight.dtype, dev, (K,))
    _check(bias, "bias", weight.dtype, dev, (N,))
    wf = torch.empty_like(weight)
    c1 = torch.empty(N, dtype=torch.float32, device=dev)
    c2 = torch.empty(N, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        st = lib.norm_gemm_fold_weights(_ptr(weight), _ptr(gamma), _ptr(beta), _ptr(bias),
                                        _ptr(wf), _ptr(c1), _ptr(c2), N, K,
                                        DTYPES[weight.dtype], _stream(dev, stream))
    if st != 0:
        raise NormGemmError(st, "norm_gemm_fold_weights")
    return wf, c1, c2


def fused_norm_gemm_folded(x: torch.Tensor, w_folded: torch.Tensor, c1: Optional[torch.Tensor],
                           c2: torch.Tensor, *, eps: float = 1e-5, norm="layernorm", act="none",
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = act(rs (x @ w_folded.T - mu c1) + c2) on the outputs of
    :func:`norm_gemm_fold_weights` (c1 may be None for RMSNorm)."""
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError("x must be a tensor with at least one dimension")
    if x.dtype not in DTYPES:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    dev = x.device
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if w_folded is None or w_folded.dim() != 2 or w_folded.shape[1] != K:
        raise ValueError(f"w_folded must be [N, {K}]")
    N = w_folded.shape[0]
    _check(x, "x", x.dtype, dev)
    _check(w_folded, "w_folded", x.dtype, dev)
    _check(c1, "c1", torch.float32, dev, (N,))
    _check(c2, "c2", torch.float32, dev, (N,))
    lead = tuple(x.shape[:-1])
    if out is None:
        out = torch.empty(lead + (N,), dtype=x.dtype, device=dev)
    _check(out, "out", x.dtype, dev, lead + (N,))
    with torch.cuda.device(dev):
        st = lib.fused_norm_gemm_folded(_ptr(x), _ptr(w_folded), _ptr(c1), _ptr(c2), _ptr(out),
                                        M, N, K, float(eps), _enum(NORMS, norm, "norm"),
                                        _enum(ACTS, act, "act"), DTYPES[x.dtype],
                                        _stream(dev, stream))
    if st != 0:
        raise NormGemmError(st, "fused_norm_gemm_folded")
    return out


def fused_gemm_norm_workspace_size(M: int, N: int) -> int:
    return int(lib.fused_gemm_norm_workspace_size(int(M), int(N)))


def fused_gemm_norm(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None, *,
                    eps: float = 1e-5, norm="rmsnorm", workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = norm_affine(x @ weight.T + bias) over each output row (gamma, beta,
    bias of length N). The fp32 sums live in ``workspace`` (uint8, at least
    :func:`fused_gemm_norm_workspace_size` bytes; twice that lets K split;
    allocated at twice that size when not given)."""
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError("x must be a tensor with at least one dimension")
    if x.dtype not in DTYPES:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    dev = x.device
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if weight is None or weight.dim() != 2 or weight.shape[1] != K:
        raise ValueError(f"weight must be [N, {K}]")
    N = weight.shape[0]
    _check(x, "x", x.dtype, dev)
    _check(weight, "weight", x.dtype, dev)
    for t, name in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _check(t, name, x.dtype, dev, (N,))
    if workspace is None:
        workspace = torch.empty(2 * fused_gemm_norm_workspace_size(M, N), dtype=torch.uint8,
                                device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on x's device")
    lead = tuple(x.shape[:-1])
    if out is None:
        out = torch.empty(lead + (N,), dtype=x.dtype, device=dev)
    _check(out, "out", x.dtype, dev, lead + (N,))
    with torch.cuda.device(dev):
        st = lib.fused_gemm_norm(_ptr(x), _ptr(weight), _ptr(bias), _ptr(gamma), _ptr(beta),
                                 _ptr(out), M, N, K, float(eps), _enum(NORMS, norm, "norm"),
                                 DTYPES[x.dtype], _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _stream(dev, stream))
    if st != 0:
        raise NormGemmError(st, "fused_gemm_norm")
    return out
