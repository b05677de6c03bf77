"""MI355X-native large-chunk TTT layer (ZipMap / LaCT fast-weight update and read).

The compute runs in libzmttt.so (hand-written HIP kernels for gfx950) behind
the C ABI of include/zm_ttt.h; this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    APPLY_THEN_UPDATE,
    BF16,
    ERR_HIP,
    ERR_INVALID_ARG,
    ERR_UNSUPPORTED,
    ERR_WORKSPACE,
    EXPORTED,
    F32,
    LIB_PATH,
    OK,
    RENORM_NONE,
    RENORM_ROW,
    STEP_GRADIENT,
    STEP_NEWTON_SCHULZ,
    UPDATE_THEN_APPLY,
    Desc,
    ZmError,
    apply,
    chunked,
    load_library,
    make_desc,
    set_profile_events,
    status_string,
    stream_step,
    update,
    update_apply,
    version,
    workspace_size,
)
