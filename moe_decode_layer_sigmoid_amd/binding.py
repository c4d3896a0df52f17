"""ctypes binding of libmoe_decode.so (the C ABI in include/moe_decode.h).

Argument marshalling only: every step of the layer runs in the HIP library.
The functions keep the C names (moe_decode_plan -> plan, moe_decode_run ->
run, ...).  Tensors are torch CUDA tensors; only their device pointers cross
the boundary, and the current torch stream is passed as the HIP stream.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_decode.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_NO_MEMORY, ERR_SCRATCH = range(6)
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_DECODE_STATIC_SCRATCH_BYTES
SCALE_FP32, SCALE_E8M0 = 0, 1
PATH_AUTO, PATH_GEMV, PATH_GROUPED, PATH_GEMV_SPLIT = 0, 1, 2, 3


PROBE_STEP = 64 << 20  # moe_decode_read_probe reads a multiple of this many bytes


class MoeDecodeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__("%s: %s (%d)" % (what, strerror(code), code))
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("shared_intermediate", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("scale_fmt", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("swiglu_limit", ctypes.c_float),
        ("routed_scaling_factor", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
    ]


class Args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "hidden", "residual", "router_w", "router_bias", "w13", "w13_scale", "w2", "w2_scale",
        "sw13", "sw13_scale", "sw2", "sw2_scale", "gamma", "out", "residual_out",
        "topk_ids", "topk_weights", "moe_out")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no
    fallback implementation)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libmoe_decode.so is not built; run `python -m moe_decode_layer_sigmoid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.moe_decode_desc_check.argtypes = [ctypes.POINTER(Desc)]
        L.moe_decode_args_check.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args), i32]
        L.moe_decode_plan.argtypes = [ctypes.POINTER(Desc), ctypes.c_int, ctypes.POINTER(vp)]
        L.moe_decode_run.argtypes = [vp, ctypes.POINTER(Args), i32, vp]
        L.moe_decode_destroy.argtypes = [vp]
        L.moe_decode_strerror.argtypes = [ctypes.c_int]
        L.moe_decode_strerror.restype = ctypes.c_char_p
        L.moe_decode_last_routes.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_decode_set_expert_events.argtypes = [vp, vp, vp]
        L.moe_decode_path_for.argtypes = [vp, i32]
        L.moe_decode_check_waits.argtypes = [vp, ctypes.POINTER(i32)]
        L.moe_decode_workspace_bytes.argtypes = [vp]
        L.moe_decode_workspace_bytes.restype = ctypes.c_size_t
        L.moe_decode_read_probe.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.moe_decode_run_static.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args), i32, vp]
        for f in ("desc_check", "args_check", "plan", "run", "destroy", "last_routes",
                  "set_expert_events", "path_for", "check_waits", "read_probe", "run_static"):
            getattr(L, "moe_decode_" + f).restype = ctypes.c_int
        _lib = L
    return _lib


EXPORTED = ["moe_decode_desc_check", "moe_decode_args_check", "moe_decode_plan",
            "moe_decode_run", "moe_decode_destroy", "moe_decode_strerror",
            "moe_decode_last_routes", "moe_decode_set_expert_events", "moe_decode_path_for",
            "moe_decode_check_waits", "moe_decode_workspace_bytes", "moe_decode_read_probe",
            "moe_decode_run_static"]


def strerror(code: int) -> str:
    return lib().moe_decode_strerror(code).decode()


def make_desc(H, E, k, I, Is, max_tokens, scale_fmt="fp32", path=PATH_AUTO, limit=7.0,
              rsf=2.5, eps=1e-5) -> Desc:
    fmt = {"fp32": SCALE_FP32, "e8m0": SCALE_E8M0}.get(scale_fmt, scale_fmt)
    return Desc(H, E, k, I, Is, max_tokens, fmt, path, limit, rsf, eps)


def desc_check(d: Desc) -> int:
    return lib().moe_decode_desc_check(ctypes.byref(d))


def args_check(d: Desc, a: Args, T: int) -> int:
    return lib().moe_decode_args_check(ctypes.byref(d), ctypes.byref(a), T)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """moe_decode_plan / moe_decode_run / moe_decode_destroy."""

    def __init__(self, desc: Desc, device: int = 0):
        self.desc = desc
        self.device = device
        self._h = ctypes.c_void_p()
        rc = lib().moe_decode_plan(ctypes.byref(desc), device, ctypes.byref(self._h))
        if rc:
            raise MoeDecodeError(rc, "moe_decode_plan")

    def close(self):
        if self._h:
            lib().moe_decode_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def make_args(self, *, hidden, residual, router_w, w13, w13_scale, w2, w2_scale, gamma,
                  out, residual_out, router_bias=None, sw13=None, sw13_scale=None, sw2=None,
                  sw2_scale=None, topk_ids=None, topk_weights=None, moe_out=None) -> Args:
        return Args(*[_ptr(t) for t in (
            hidden, residual, router_w, router_bias, w13, w13_scale, w2, w2_scale, sw13,
            sw13_scale, sw2, sw2_scale, gamma, out, residual_out, topk_ids, topk_weights,
            moe_out)])

    def run_args(self, args: Args, T: int, stream=None) -> None:
        rc = lib().moe_decode_run(self._h, ctypes.byref(args), T, _stream(stream))
        if rc:
            raise MoeDecodeError(rc, "moe_decode_run")

    def run(self, T: int, stream=None, **tensors) -> None:
        """moe_decode_run with the tensors named as in moe_decode_args."""
        self.run_args(self.make_args(**tensors), T, stream)

    def last_routes(self, T, counts=None, offsets=None, perm=None, touched=None,
                    n_touched=None, stream=None) -> None:
        rc = lib().moe_decode_last_routes(self._h, T, _ptr(counts), _ptr(offsets), _ptr(perm),
                                          _ptr(touched), _ptr(n_touched), _stream(stream))
        if rc:
            raise MoeDecodeError(rc, "moe_decode_last_routes")

    def set_expert_events(self, begin, end) -> None:
        b = None if begin is None else begin.cuda_event
        e = None if end is None else end.cuda_event
        rc = lib().moe_decode_set_expert_events(self._h, b, e)
        if rc:
            raise MoeDecodeError(rc, "moe_decode_set_expert_events")

    def path_for(self, T: int) -> int:
        return lib().moe_decode_path_for(self._h, T)

    def check_waits(self) -> bool:
        """True when a bounded wait of a run gave up since the
        last check (synchronises the device; clears the flag)."""
        flag = ctypes.c_int32(0)
        rc = lib().moe_decode_check_waits(self._h, ctypes.byref(flag))
        if rc:
            raise MoeDecodeError(rc, "moe_decode_check_waits")
        return bool(flag.value)

    def workspace_bytes(self) -> int:
        return lib().moe_decode_workspace_bytes(self._h)


def read_probe(buf, nbytes: int, sink, stream=None) -> None:
    """moe_decode_read_probe: one streaming read of `nbytes` of `buf` (a
    measurement kernel for the benchmark's read ceiling)."""
    rc = lib().moe_decode_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_read_probe")


def run_static(desc: Desc, T: int, stream=None, **tensors) -> None:
    """moe_decode_run_static: the layer without a plan, its workspace in the
    library's static scratch array (no device allocation)."""
    fields = {n: None for n, _ in Args._fields_}
    fields.update(tensors)
    args = Args(*[_ptr(fields[n]) for n, _ in Args._fields_])
    rc = lib().moe_decode_run_static(ctypes.byref(desc), ctypes.byref(args), T, _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_run_static")
