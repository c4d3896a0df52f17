"""The C-ABI library on the host (no GPU): it loads, exports every function
include/*.h declares, and rejects bad descriptors and arguments before any
launch."""

import ctypes
import glob
import os
import re

import pytest
from hypothesis import given, settings, strategies as st

import moe_decode_layer_sigmoid_amd as md

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(moe_decode_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = md.lib()
    names = declared_functions()
    assert "moe_decode_plan" in names and "moe_decode_run" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(md.EXPORTED) == names


def good_desc(**kw):
    base = dict(H=4096, E=128, k=8, I=1536, Is=1536, max_tokens=16)
    base.update(kw)
    return md.make_desc(base["H"], base["E"], base["k"], base["I"], base["Is"],
                        base["max_tokens"])


def test_desc_check_codes():
    assert md.desc_check(good_desc()) == md.OK
    assert md.desc_check(good_desc(Is=0)) == md.OK
    for kw, code in [
        (dict(H=4000), md.ERR_UNSUPPORTED),
        (dict(I=100), md.ERR_UNSUPPORTED),
        (dict(Is=64), md.ERR_UNSUPPORTED),
        (dict(H=8320), md.ERR_UNSUPPORTED),
        (dict(k=17, E=64), md.ERR_UNSUPPORTED),
        (dict(k=9, E=8), md.ERR_UNSUPPORTED),
        (dict(E=1025), md.ERR_UNSUPPORTED),
        (dict(max_tokens=257), md.ERR_UNSUPPORTED),
        (dict(H=0), md.ERR_INVALID_ARG),
        (dict(max_tokens=0), md.ERR_INVALID_ARG),
        (dict(Is=-128), md.ERR_INVALID_ARG),
    ]:
        assert md.desc_check(good_desc(**kw)) == code, kw
    d = good_desc()
    d.scale_fmt = 7
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    d = good_desc()
    d.path = 9
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    d = good_desc()
    d.swiglu_limit = 0.0
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    d = good_desc()
    d.rms_eps = float("nan")
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    assert md.lib().moe_decode_desc_check(None) == md.ERR_INVALID_ARG


def test_dense_layer_descriptors():
    """No routed experts (E = 0, k = 0): a dense layer whose MLP sits in the
    shared-expert slot; it needs that slot, and a MoE layer needs k and I."""
    d = good_desc()
    d.num_experts, d.top_k, d.intermediate = 0, 0, 0
    assert md.desc_check(d) == md.OK
    d.top_k = 1
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    d.top_k, d.shared_intermediate = 0, 0
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    d = good_desc()
    d.top_k = 0
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    d = good_desc()
    d.intermediate = 0
    assert md.desc_check(d) == md.ERR_INVALID_ARG
    # a dense layer's run needs no router or routed-expert pointers
    d = good_desc()
    d.num_experts, d.top_k, d.intermediate = 0, 0, 0
    none = dict(router_w=None, w13=None, w13_scale=None, w2=None, w2_scale=None)
    assert md.args_check(d, full_args(**none), 1) == md.OK
    assert md.args_check(d, full_args(sw13=None, **none), 1) == md.ERR_INVALID_ARG


def full_args(**kw):
    names = [f for f, _ in md.Args._fields_]
    vals = {n: 0x10000 * (i + 1) for i, n in enumerate(names)}
    vals["router_bias"] = None
    vals["topk_ids"] = None
    vals["topk_weights"] = None
    vals.update(kw)
    return md.Args(*[vals[n] for n in names])


def test_args_check_codes():
    d = good_desc()
    assert md.args_check(d, full_args(), 1) == md.OK
    assert md.args_check(d, full_args(), 0) == md.OK
    assert md.args_check(d, full_args(), 16) == md.OK
    assert md.args_check(d, full_args(), 17) == md.ERR_INVALID_ARG
    assert md.args_check(d, full_args(), -1) == md.ERR_INVALID_ARG
    for n in ["hidden", "residual", "router_w", "w13", "w13_scale", "w2", "w2_scale", "gamma",
              "out", "residual_out", "sw13", "sw2_scale"]:
        assert md.args_check(d, full_args(**{n: None}), 1) == md.ERR_INVALID_ARG, n
    # no shared expert: shared pointers may be NULL
    d0 = good_desc(Is=0)
    assert md.args_check(d0, full_args(sw13=None, sw13_scale=None, sw2=None, sw2_scale=None),
                         1) == md.OK
    # misaligned vector operand
    assert md.args_check(d, full_args(w13=0x10008), 1) == md.ERR_INVALID_ARG
    # out may not alias an input; residual_out may alias residual only
    a = full_args()
    assert md.args_check(d, full_args(out=a.hidden), 1) == md.ERR_INVALID_ARG
    assert md.args_check(d, full_args(residual_out=a.residual), 1) == md.OK
    assert md.args_check(d, full_args(residual_out=a.hidden), 1) == md.ERR_INVALID_ARG
    # the finalized MoE output is optional, aligned, and aliases nothing
    assert md.args_check(d, full_args(moe_out=None), 1) == md.OK
    assert md.args_check(d, full_args(moe_out=0x10008), 1) == md.ERR_INVALID_ARG
    for n in ["hidden", "residual", "out", "residual_out"]:
        assert md.args_check(d, full_args(moe_out=getattr(a, n)), 1) == md.ERR_INVALID_ARG, n


def test_strerror_and_null_plan():
    assert md.strerror(md.OK) == "ok"
    assert "invalid" in md.strerror(md.ERR_INVALID_ARG)
    assert md.strerror(99) == "unknown status"
    lib = md.lib()
    assert lib.moe_decode_destroy(None) == md.OK
    assert lib.moe_decode_run(None, None, 1, None) == md.ERR_INVALID_ARG
    assert lib.moe_decode_workspace_bytes(None) == 0
    out = ctypes.c_void_p(1)
    assert lib.moe_decode_plan(None, 0, ctypes.byref(out)) == md.ERR_INVALID_ARG
    assert not out.value


def _expected_desc_code(H, E, k, I, Is, T, fmt, path, limit, eps):
    """The descriptor rules as include/moe_decode.h states them: INVALID_ARG
    for a non-positive or negative size, a bad enum or constant, or a layer
    that is neither a MoE layer (k >= 1, I > 0) nor a dense one (E = k = 0
    with a shared-expert slot); UNSUPPORTED outside the size limits."""
    if H <= 0 or E < 0 or k < 0 or I < 0 or Is < 0 or T <= 0:
        return md.ERR_INVALID_ARG
    if (E == 0 and (k != 0 or Is == 0)) or (E > 0 and (k == 0 or I == 0)):
        return md.ERR_INVALID_ARG
    if fmt not in (md.SCALE_FP32, md.SCALE_E8M0) or path not in (0, 1, 2, 3):
        return md.ERR_INVALID_ARG
    if not limit > 0 or not eps >= 0:
        return md.ERR_INVALID_ARG
    if H % 128 or I % 128 or Is % 128 or max(H, I, Is) > 8192:
        return md.ERR_UNSUPPORTED
    if k > 16 or k > E or E > 1024 or T > 256:
        return md.ERR_UNSUPPORTED
    return md.OK


SIZES = [-128, 0, 64, 100, 128, 1536, 4096, 8192, 8320]


@settings(max_examples=400, deadline=None)
@given(H=st.sampled_from(SIZES), E=st.sampled_from([-1, 0, 1, 8, 128, 1024, 1025]),
       k=st.sampled_from([-1, 0, 1, 2, 8, 16, 17]), I=st.sampled_from(SIZES),
       Is=st.sampled_from(SIZES), T=st.sampled_from([-1, 0, 1, 16, 256, 257]),
       fmt=st.sampled_from([0, 1, 2, -1]), path=st.sampled_from([0, 1, 2, 3, 4, -1]),
       limit=st.sampled_from([7.0, 0.0, -1.0, float("nan")]),
       eps=st.sampled_from([1e-5, 0.0, -1e-6, float("nan")]))
def test_desc_check_matches_documented_rules(H, E, k, I, Is, T, fmt, path, limit, eps):
    """moe_decode_desc_check on descriptors drawn around every limit agrees
    with the rules the header documents."""
    d = md.make_desc(H, E, k, I, Is, T, scale_fmt=fmt, path=path, limit=limit, eps=eps)
    assert md.desc_check(d) == _expected_desc_code(H, E, k, I, Is, T, fmt, path, limit, eps)
