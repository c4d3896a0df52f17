"""The MFMA kernels stage weights HBM -> LDS with loads that write LDS
directly (global_load_lds).  The compiler does not order later LDS reads
after such loads, so each kernel must wait for them (s_waitcnt vmcnt(0))
before it reads the staged block.  A build where a ds_read follows those
loads with no full wait in between reads stale LDS; this happened once with
the same source, when the kernels were reorganised and the compiler moved
its wait below the reads.

This compiles experts_mfma.hip and router.hip for gfx950 to assembly (no GPU
needed) and checks every kernel that stages in program order.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_decode_layer_sigmoid_amd", "csrc")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _check_source(tmp_path, src, pattern, min_kernels):
    from moe_decode_layer_sigmoid_amd import build as hip_build

    out = tmp_path / (src + ".s")
    cmd = [_hipcc(), *hip_build.FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    cmd = [c for c in cmd if c != "-fPIC"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-2000:]
    asm = out.read_text()
    kernels = re.findall(r"^(_Z\S*(?:%s)\S*):" % pattern, asm, re.M)
    assert len(kernels) >= min_kernels, kernels
    checked = 0
    for name in kernels:
        body = asm[asm.index(name + ":"):asm.index(".Lfunc_end", asm.index(name + ":"))]
        pending = False
        for line in (x.strip() for x in body.splitlines()):
            if line.startswith("global_load_lds"):
                pending = True
            elif line.startswith("s_waitcnt") and "vmcnt(0)" in line:
                pending = False
            elif line.startswith("ds_read"):
                assert not pending, "%s: %s before its staged loads are waited for" % (name, line)
        checked += "global_load_lds" in body
    return checked


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_staged_lds_reads_wait_for_their_loads(tmp_path):
    assert _check_source(tmp_path, "experts_mfma.hip", "mfma_kernel|chain_kernel", 10) >= 10


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_router_staged_token_rows_wait_for_their_loads(tmp_path):
    """The matrix-core router stages each round's token rows the same way."""
    assert _check_source(tmp_path, "router.hip", "router_mfma_kernel", 1) == 1
