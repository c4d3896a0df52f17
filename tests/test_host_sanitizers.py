"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C oracle run over every branch it has (oracle_driver.c), and the
C-ABI's host-side checks and argument rejections (abi_driver.c) linked
against the library's sources built with the sanitizers on the host pass
only.  No device is touched; a sanitizer report fails the test through the
driver's exit status."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from moe_decode_layer_sigmoid_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return res.returncode, res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "moe_oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=SAN_ENV, timeout=300)
    assert rc == 0, out
    assert "FAIL" not in out and out.count(": ok") == 5, out


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    try:
        hipcc = lib_build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    csrc = lib_build.CSRC
    # the library's flags with the sanitizers added to the host pass only
    flags = [f for f in lib_build.FLAGS if f != "-O3"] + ["-O1"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    jobs = []
    for src in lib_build.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        jobs.append([hipcc, *flags, *san, *inc, "-c", os.path.join(csrc, src), "-o", obj])
    for nj in lib_build.CHAIN_NJG:
        obj = str(tmp_path / ("chain_njg%d.o" % nj))
        jobs.append([hipcc, *flags, *san, *inc, "-DMOE_CHAIN_NJG=%d" % nj, "-c",
                     os.path.join(csrc, "experts_chain.hip"), "-o", obj])
    jobs.append([hipcc, *san, *inc, "-x", "c", "-c", os.path.join(HERE, "abi_driver.c"),
                 "-o", str(tmp_path / "driver.o")])
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, jobs))
    for cmd, (rc, out) in zip(jobs, results):
        assert rc == 0, " ".join(cmd) + "\n" + out
    exe = str(tmp_path / "abi_san")
    objs = [j[j.index("-o") + 1] for j in jobs]
    rc, out = _run([hipcc, "--offload-arch=" + lib_build.ARCH, *san, *objs, "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=SAN_ENV, timeout=300)
    assert rc == 0, out
    assert "abi checks: ok" in out, out
