"""CPU check of the generated gfx950 code of the MX prefill GEMMs (mx_gemm.hip).

Their activation tiles are loaded into LDS by inline-asm LDS-DMA buffer loads, invisible to
the compiler, so each K step waits for its tile with an explicit `s_waitcnt vmcnt(N)` before
the workgroup barrier.  That is correct only while at least N vector-memory loads are issued
after the awaited tile (loads complete in issue order).  The tile of step s is the
second-newest LDS-DMA group when step s begins (the tile of step s + 1 was issued after it).
If the compiler drops loads (for instance weight loads whose data no MFMA uses) the count
shrinks and the wait no longer covers the tile: the kernels would read stale LDS.  This test
compiles the source to assembly and checks every such wait, in text order, in every
instantiation.  It needs hipcc (present in the build image), not a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_moe_softmax_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.slow


def _asm(tmp_path):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "mx_gemm.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-Wno-inline-asm", "-mllvm", "-pragma-unroll-threshold=1000000",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "--cuda-device-only", "-S",
           os.path.join(CSRC, "mx_gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _barrier_waits(body):
    """(N, loads issued after the second-newest LDS-DMA group) for every vmcnt wait that
    directly precedes an s_barrier, scanning the kernel's text in order."""
    lines = [ln.strip() for ln in body.splitlines()]
    groups, vm, prev_dma, res = [], 0, False, []
    for i, ln in enumerate(lines):
        if ln.startswith("buffer_load") or ln.startswith("global_load"):
            vm += 1
            is_dma = ln.endswith(" lds")
            if is_dma:
                if prev_dma:
                    groups[-1] = vm
                else:
                    groups.append(vm)
            prev_dma = is_dma
        m = re.match(r"s_waitcnt vmcnt\((\d+)\)", ln)
        if m and i + 1 < len(lines) and lines[i + 1] == "s_barrier" and len(groups) >= 2:
            res.append((int(m.group(1)), vm - groups[-2]))
    return res


def test_mx_gemm_tile_waits_cover_the_awaited_tile(tmp_path):
    txt = _asm(tmp_path)
    kernels = sorted(set(re.findall(r"^(_Z\w*mx_gemm_kernel\w*):", txt, re.M)))
    assert len(kernels) == 4, kernels   # gate/up and down, tiled and row-major
    for k in kernels:
        body = re.search(r"^" + re.escape(k) + r":[^\n]*\n(.*?)s_endpgm", txt, re.S | re.M).group(1)
        assert " lds" in body, f"{k}: no LDS-DMA loads"
        waits = _barrier_waits(body)
        assert len(waits) >= 8, f"{k}: expected one explicit wait per K step, found {len(waits)}"
        bad = [w for w in waits if w[0] > w[1]]
        assert not bad, f"{k}: waits that do not cover their tile (vmcnt, loads after it): {bad[:5]}"
        # the steady-state wait: 8 weight loads of the previous step + 3 tile loads of the next
        assert max(w[0] for w in waits) == 11, f"{k}: {sorted(set(waits))}"
