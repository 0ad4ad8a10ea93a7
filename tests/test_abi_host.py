"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and every validation error returns its status without a
kernel launch (all failing calls below return before any HIP call)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import norm_gemm_amd as ng

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "norm_gemm.h")

OK, NULL, SHAPE, ENUM, EPS, ALIAS, WORKSPACE, UNSUP, ALIGN, HIP, SCRATCH = \
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10

# Fake device addresses: validation compares them as integers and never
# dereferences them; each failing call returns before any HIP call. Where a
# GPU is visible these calls are skipped, so that a validation regression can
# never launch a kernel on such addresses.
X, G, B, W, BI, Y, WS = (0x10000000 * (i + 1) for i in range(7))

import torch  # noqa: E402

no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                 reason="fake-address validation runs only where no GPU is visible")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(ng.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ng.LIBRARY_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(ng.lib, name)


def test_abi_version_and_status_strings():
    assert ng.norm_gemm_abi_version() == 5
    for s in (OK, NULL, SHAPE, ENUM, EPS, ALIAS, WORKSPACE, UNSUP, ALIGN, HIP, SCRATCH):
        assert ng.norm_gemm_status_string(s)
    assert ng.norm_gemm_status_string(12345) == "unknown status"


def test_workspace_size():
    assert ng.fused_ffn_workspace_size(512, 49152, 0) == 512 * 49152 * 2
    assert ng.fused_ffn_workspace_size(3, 5, 1) == 256
    assert ng.fused_ffn_workspace_size(0, 5, 0) == 0
    assert ng.fused_ffn_workspace_size(3, 5, 7) == 0


def gemm(x=X, g=G, b=B, w=W, bias=BI, y=Y, M=4, N=8, K=16, eps=1e-5, norm=1, act=0, dtype=0):
    return ng.lib.fused_norm_gemm(x, g, b, w, bias, y, M, N, K, eps, norm, act, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL),
    (dict(norm=3), ENUM), (dict(norm=-1), ENUM), (dict(act=4), ENUM), (dict(dtype=2), ENUM),
    (dict(M=0), SHAPE), (dict(N=0), SHAPE), (dict(K=0), SHAPE), (dict(M=-5), SHAPE),
    (dict(K=2 ** 31), SHAPE), (dict(M=2 ** 31 - 1, N=2 ** 31 - 1, K=2 ** 31 - 1), SHAPE),
    (dict(eps=float("nan")), EPS), (dict(eps=float("inf")), EPS), (dict(eps=-1e-6), EPS),
    (dict(x=X + 1), ALIGN), (dict(g=G + 1), ALIGN), (dict(bias=BI + 3), ALIGN), (dict(y=Y + 1), ALIGN),
    (dict(y=X), ALIAS), (dict(y=X + 2 * 4 * 16 - 2), ALIAS), (dict(y=W + 2), ALIAS),
    (dict(y=G), ALIAS), (dict(y=BI - 2), ALIAS),
])
@no_gpu_only
def test_fused_norm_gemm_validation_errors(kw, status):
    assert gemm(**kw) == status


@no_gpu_only
def test_eps_is_ignored_without_norm_but_enums_are_not():
    # norm NONE ignores eps, so a NaN eps is not an error there; use a
    # failing alias to stop before any launch.
    assert gemm(norm=0, eps=float("nan"), y=X) == ALIAS
    assert gemm(norm=0, eps=float("nan"), act=5) == ENUM


def ffn(x=X, g=G, b=B, w1=W, b1=BI, w2=0x90000000, b2=0xA0000000, y=Y, M=4, K=16, F=32, N=8,
        eps=1e-5, norm=1, act=1, dtype=0, ws=WS, wsb=4 * 32 * 2):
    return ng.lib.fused_ffn(x, g, b, w1, b1, w2, b2, y, M, K, F, N, eps, norm, act, dtype,
                            ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w2=None), NULL), (dict(x=None), NULL), (dict(act=9), ENUM), (dict(F=0), SHAPE),
    (dict(eps=-1.0), EPS), (dict(ws=WS + 1), ALIGN), (dict(y=0x90000000), ALIAS),
    (dict(ws=None), WORKSPACE), (dict(wsb=4 * 32 * 2 - 1), WORKSPACE),
    (dict(ws=X), ALIAS), (dict(ws=0x90000000 + 64), ALIAS), (dict(ws=Y), ALIAS),
])
@no_gpu_only
def test_fused_ffn_validation_errors(kw, status):
    assert ffn(**kw) == status


# A workspace large enough for the split-K partials of y (h, 256 bytes here,
# then 8 M N bytes) is alias-checked over all of them; a smaller one only
# over h.
@no_gpu_only
def test_fused_ffn_split_k_workspace_is_alias_checked():
    assert ffn(wsb=256 + 8 * 4 * 8, y=WS + 300) == ALIAS
    assert ffn(wsb=256 + 8 * 4 * 8, x=WS + 400) == ALIAS
    assert gffn(wsb=3 * 4 * 32 * 2, y=WS + 700) == ALIAS


def gffn(x=X, g=G, b=B, w1=W, b1=BI, w2=0x90000000, b2=0xA0000000, y=Y, M=4, K=16, F=32, N=8,
         eps=1e-5, norm=1, act=1, dtype=0, ws=WS, wsb=3 * 4 * 32 * 2):
    return ng.lib.fused_gated_ffn(x, g, b, w1, b1, w2, b2, y, M, K, F, N, eps, norm, act, dtype,
                                  ws, wsb, None)


def test_gated_ffn_workspace_size():
    assert ng.fused_gated_ffn_workspace_size(512, 28672, 0) == 3 * 512 * 28672 * 2
    assert ng.fused_gated_ffn_workspace_size(3, 5, 1) == 256
    assert ng.fused_gated_ffn_workspace_size(0, 5, 0) == 0
    assert ng.fused_gated_ffn_workspace_size(3, 5, 7) == 0
    assert ng.fused_gated_ffn_workspace_size(1, 2 ** 30, 0) == 0


# W1 is [2F, K] (2 KB here) and b1 [2F]: overlaps with their second halves
# are caught; the workspace must hold 3 M F elements.
@pytest.mark.parametrize("kw,status", [
    (dict(w1=None), NULL), (dict(act=9), ENUM), (dict(F=0), SHAPE), (dict(F=2 ** 30), SHAPE),
    (dict(wsb=3 * 4 * 32 * 2 - 1), WORKSPACE), (dict(wsb=4 * 32 * 2), WORKSPACE),
    (dict(y=W + 2 * 32 * 16 * 2 - 64), ALIAS), (dict(y=BI + 2 * 32 * 2 - 2), ALIAS),
    (dict(ws=W + 2 * 32 * 16 * 2 - 256), ALIAS), (dict(ws=Y - 512), ALIAS),
])
@no_gpu_only
def test_fused_gated_ffn_validation_errors(kw, status):
    assert gffn(**kw) == status


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 8, dtype=torch.float16)
    w = torch.zeros(3, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        ng.fused_norm_gemm(x, w)
    with pytest.raises(ValueError):
        ng.fused_norm_gemm(x.float(), w)


def ffn_noalloc(x=X, g=G, b=B, w1=W, b1=BI, w2=0x90000000, b2=0xA0000000, y=Y, M=4, K=16, F=32,
                N=8, eps=1e-5, norm=1, act=1, dtype=0):
    return ng.lib.fused_ffn_noalloc(x, g, b, w1, b1, w2, b2, y, M, K, F, N, eps, norm, act, dtype,
                                    None)


# Every status below is returned before any HIP call (argument checks, then
# the scratch size), so these run only where no GPU is visible.
@pytest.mark.parametrize("kw,status", [
    (dict(w2=None), NULL), (dict(act=9), ENUM), (dict(F=0), SHAPE), (dict(eps=-1.0), EPS),
    (dict(y=X + 1), ALIGN), (dict(y=0x90000000), ALIAS),
    # h = M F 2 bytes: 64 MiB + 256 bytes is one 256-byte block past the array
    (dict(M=512, F=65536 + 1, K=16), SCRATCH),
])
@no_gpu_only
def test_fused_ffn_noalloc_validation_errors(kw, status):
    assert ffn_noalloc(**kw) == status


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER, encoding="utf-8").read()
    assert "#define NG_FFN_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert ng.NOALLOC_SCRATCH_BYTES == 64 << 20


def fold(w=W, g=G, b=B, bias=BI, wf=0x90000000, c1=0xA0000000, c2=0xB0000000, N=8, K=16,
         dtype=0):
    return ng.lib.norm_gemm_fold_weights(w, g, b, bias, wf, c1, c2, N, K, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), NULL), (dict(wf=None), NULL), (dict(c1=None), NULL), (dict(c2=None), NULL),
    (dict(dtype=3), ENUM), (dict(N=0), SHAPE), (dict(K=2 ** 31), SHAPE),
    (dict(wf=0x90000001), ALIGN), (dict(c1=0xA0000002), ALIGN), (dict(g=G + 1), ALIGN),
    (dict(wf=W + 2), ALIAS), (dict(c1=G), ALIAS), (dict(c2=0xA0000000 + 16), ALIAS),
    (dict(c2=0x90000000 + 8 * 16 * 2 - 4), ALIAS),
])
@no_gpu_only
def test_fold_weights_validation_errors(kw, status):
    assert fold(**kw) == status


def folded(x=X, wf=W, c1=0xA0000000, c2=0xB0000000, y=Y, M=4, N=8, K=16, eps=1e-5, norm=1,
           act=0, dtype=0):
    return ng.lib.fused_norm_gemm_folded(x, wf, c1, c2, y, M, N, K, eps, norm, act, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(c2=None), NULL), (dict(c1=None, norm=1), NULL),
    (dict(norm=0), ENUM), (dict(norm=3), ENUM), (dict(act=7), ENUM), (dict(M=0), SHAPE),
    (dict(eps=-1.0), EPS), (dict(y=Y + 1), ALIGN), (dict(c2=0xB0000001), ALIGN),
    (dict(y=X), ALIAS), (dict(y=0xB0000000 - 4), ALIAS), (dict(y=W + 6), ALIAS),
    # unaligned x or K % 8 != 0: the tiled kernel cannot serve the call
    (dict(x=X + 2), UNSUP), (dict(K=20), UNSUP),
])
@no_gpu_only
def test_fused_norm_gemm_folded_validation_errors(kw, status):
    assert folded(**kw) == status


@no_gpu_only
def test_folded_rmsnorm_does_not_need_c1():
    # RMSNorm ignores c1, so a NULL c1 is valid; K % 8 != 0 then stops the
    # call before any launch
    assert folded(c1=None, norm=2, K=20) == UNSUP


def gnorm(x=X, w=W, bias=BI, g=G, b=B, y=Y, M=4, N=8, K=16, eps=1e-5, norm=2, dtype=0, ws=WS,
          wsb=256):
    return ng.lib.fused_gemm_norm(x, w, bias, g, b, y, M, N, K, eps, norm, dtype, ws, wsb, None)


def test_gemm_norm_workspace_size():
    assert ng.fused_gemm_norm_workspace_size(512, 8192) == 4 * 512 * 8192
    assert ng.fused_gemm_norm_workspace_size(3, 5) == 256
    assert ng.fused_gemm_norm_workspace_size(0, 5) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(y=None), NULL), (dict(norm=0), ENUM), (dict(dtype=2), ENUM),
    (dict(N=0), SHAPE), (dict(eps=float("nan")), EPS), (dict(ws=WS + 8), ALIGN),
    (dict(g=G + 1), ALIGN), (dict(y=X + 16), ALIAS), (dict(y=G - 8), ALIAS),
    (dict(ws=None), WORKSPACE), (dict(wsb=255), WORKSPACE), (dict(ws=Y), ALIAS),
    (dict(ws=W + 32), ALIAS),
    # a workspace of two planes is alias-checked over both
    (dict(wsb=512, y=WS + 300), ALIAS),
    # unaligned x or K % 8 != 0: the tiled kernel cannot serve the call
    (dict(x=X + 2), UNSUP), (dict(K=12), UNSUP),
])
@no_gpu_only
def test_fused_gemm_norm_validation_errors(kw, status):
    assert gnorm(**kw) == status
