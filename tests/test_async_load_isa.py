"""The prefill kernels issue their x / gamma / beta register loads as inline asm
(the compiler does not count them) and hands the destination registers
through an explicit ``s_waitcnt vmcnt`` statement before any use. The
hardware writes those registers whenever the load returns, so no instruction
may read or write them on any path between the load and the next vmcnt
wait: otherwise a copy would read stale data, or a reused register would be
overwritten late. This compiles the kernel to gfx950 assembly (no GPU
needed) and checks that property on every control-flow path of every
instantiation of both tiled kernels.
"""
import os
import re
import shutil
import subprocess

import pytest

import importlib.util

_spec = importlib.util.spec_from_file_location(
    "_norm_gemm_amd_build",
    os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "norm_gemm_amd", "build.py"))
nb = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(nb)

HIPCC = nb.HIPCC


def _vregs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def async_load_hazards(asm_lines, kernel_pattern):
    """(loads checked, list of hazards) for register-destination
    global_load_dwordx4 in kernels whose symbol matches kernel_pattern."""
    lines = [ln.split(";")[0].rstrip() for ln in asm_lines]
    starts = [(i, ln.split(":")[0]) for i, ln in enumerate(lines) if re.match(r"^_Z\S+:", ln)]
    loads, hazards = 0, []
    for ki, (k0, name) in enumerate(starts):
        if not re.search(kernel_pattern, name):
            continue
        k1 = starts[ki + 1][0] if ki + 1 < len(starts) else len(lines)
        labels = {}
        for i in range(k0, k1):
            m = re.match(r"^(\.LBB\w+):", lines[i])
            if m:
                labels[m.group(1)] = i
        for i in range(k0, k1):
            m = re.match(r"\s+global_load_dwordx4 (v\[\d+:\d+\]),", lines[i])
            if not m:
                continue
            loads += 1
            dst = _vregs(m.group(1))
            seen, stack = set(), [i + 1]
            while stack:
                j = stack.pop()
                while j < k1 and j not in seen:
                    seen.add(j)
                    t = lines[j]
                    if re.match(r"\s+s_waitcnt\b.*vmcnt", t) or re.match(r"\s+s_endpgm", t):
                        break
                    if _vregs(t) & dst and not re.match(r"\s+global_load_dwordx4", t):
                        hazards.append((name, i, j, t.strip()))
                    mb = re.match(r"\s+s_branch (\.LBB\w+)", t)
                    if mb:
                        j = labels[mb.group(1)]
                        continue
                    mc = re.match(r"\s+s_cbranch_\w+ (\.LBB\w+)", t)
                    if mc:
                        stack.append(labels[mc.group(1)])
                    j += 1
    return loads, hazards


def test_checker_finds_a_planted_hazard():
    asm = ["_Zk:", "\tglobal_load_dwordx4 v[8:11], v1, s[0:1]", "\ts_cbranch_scc1 .LBB0_2",
           "\tv_mov_b32 v2, v3", ".LBB0_2:", "\tv_add_u32 v4, v9, v5", "\ts_waitcnt vmcnt(0)",
           "\tv_mov_b32 v8, 0", "\ts_endpgm"]
    loads, hz = async_load_hazards(asm, "_Zk")
    assert loads == 1 and len(hz) == 1 and "v9" in hz[0][3]


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("source,kernel", [("prefill_lds.hip", "prefill_lds_kernel"),
                                           ("prefill_wide.hip", "prefill_wide_kernel")])
def test_prefill_async_loads_untouched_until_waited(tmp_path, source, kernel):
    out = tmp_path / (source + ".s")
    cmd = [HIPCC, *nb.HIP_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(nb.CSRC, source), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    loads, hz = async_load_hazards(out.read_text().splitlines(), kernel)
    assert loads > 0
    assert not hz, hz[:5]
