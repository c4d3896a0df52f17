"""bench.py names the kernel it times (and prices its bytes) from copies of a
few of the library's launch constants: the token limits of the chain and
merged launches, the gate_up MFMA tiles, and the mean tokens per expert from
which the routed launches take two 16-token groups per pass.  A copy that
drifts from the source makes bench.py time or price the wrong kernel, so
this reads each constant from the C++ sources and compares."""

import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_decode_layer_sigmoid_amd", "csrc")


def _src(name):
    with open(os.path.join(CSRC, name)) as f:
        return f.read()


def _const(text, name):
    m = re.search(r"\b%s\s*=\s*(\d+)\s*[;,]" % name, text)
    assert m, "constant %s not found" % name
    return int(m.group(1))


def test_token_limits_match_library():
    launch = _src("launch.h")
    assert bench.MERGE_SHARED_MAX_TOKENS == _const(launch, "kMergeSharedMaxTokens")
    assert bench.CHAIN_MAX_TOKENS == _const(launch, "kChainMaxTokens")
    assert bench.FUSED_BOUNDARY_MAX_TOKENS == _const(launch, "kFusedBoundaryMaxTokens")


def test_mfma_tile_matches_library():
    mfma = _src("experts_mfma.hip")
    ns, u, gr = (int(x) for x in bench.MFMA_GATE_UP_TILE.split(","))
    assert (ns, u, gr) == (_const(mfma, "kNsGu"), _const(mfma, "kUGu"), _const(mfma, "kGR"))
    ns_r, u_r = (int(x) for x in bench.MFMA_ROUTED_TILE.split(","))
    assert (ns_r, u_r) == (ns, u)
    assert bench.GR2_MIN_MEAN == _const(mfma, "kGr2MinMean")
    assert bench.SHARED_ACT_MIN_MEAN == _const(mfma, "kSharedActMinMean")
    assert re.search(r"d\.T \* d\.k >= kSharedActMinMean \* d\.E", mfma)
    assert bench.SHARED_ACT_MIN_MEAN1 == _const(mfma, "kSharedActMinMean1")
    assert bench.MFMA_GATE_UP_WIDE_NS == _const(mfma, "kNsGuWide")
    assert re.search(r"d\.T \* d\.k >= kSharedActMinMean1 \* d\.E", mfma)
    # a dense layer's gate_up kernel takes up to kDenseMaxGroups 16-token groups
    assert bench.DENSE_MAX_GROUPS == _const(mfma, "kDenseMaxGroups")
    assert "dense_gate_up_mfma_kernel" in mfma
    # bench.py names that kernel's blocks per round by the same rule
    assert re.search(r"constexpr int NB = GR == kDenseMaxGroups \? 1 : 2;", mfma)
    # the rule bench.py applies is the library's: T * k >= kGr2MinMean * E
    assert re.search(r"d\.T \* d\.k >= kGr2MinMean \* d\.E", mfma)


def test_bench_refuses_several_gpus():
    """The layer runs on one GPU: asked for more, bench.py says so and exits
    with an error before it touches a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
