"""MI355X (gfx950) decode-step MoE layer with a sigmoid router.

The layer runs in hand-written HIP kernels behind the C ABI declared in
include/moe_decode.h (libmoe_decode.so, built in-tree by
``python -m moe_decode_layer_sigmoid_amd.build``).  This package is its thin
Python binding; PyTorch only provides device memory and streams.
"""

from .binding import (  # noqa: F401
    Args,
    Desc,
    MoeDecodeError,
    Plan,
    EXPORTED,
    LIB_PATH,
    OK,
    ERR_HIP,
    ERR_INVALID_ARG,
    ERR_NO_MEMORY,
    ERR_SCRATCH,
    STATIC_SCRATCH_BYTES,
    ERR_UNSUPPORTED,
    PATH_AUTO,
    PATH_GEMV,
    PATH_GROUPED,
    PATH_GEMV_SPLIT,
    SCALE_E8M0,
    SCALE_FP32,
    args_check,
    desc_check,
    lib,
    make_desc,
    read_probe,
    run_static,
    strerror,
    PROBE_STEP,
)
