"""MI355X-native (gfx950) implementation of Moshi's RQ-Transformer frame step.

The computation lives in the HIP library ``libmoshi.so`` (C ABI in
include/moshi.h); this package holds its ctypes binding and build script.
"""
from .binding import (  # noqa: F401
    MOSHI_BF16,
    MOSHI_Q8,
    MOSHI_STEP_TEXT_ONLY,
    MOSHI_DEVICE_PTRS,
    MOSHI_F32,
    MOSHI_TF_FILL_KV,
    MOSHI_TF_SKIP_DEPTH,
    Moshi,
    MoshiError,
    config_struct,
    lib,
    moshi_check_config,
    moshi_create,
    moshi_delay_codes,
    moshi_destroy,
    moshi_forward_teacher_forced,
    moshi_init_weights,
    moshi_last_error,
    moshi_loss,
    moshi_position,
    moshi_read_q8,
    moshi_tts_text,
    moshi_set_sampling,
    moshi_rvq_work_bytes,
    moshi_rvq_encode,
    moshi_rvq_decode,
    moshi_reset,
    moshi_step,
    moshi_sync,
    moshi_time_kernel,
    moshi_undelay_codes,
    moshi_workspace_bytes,
)
