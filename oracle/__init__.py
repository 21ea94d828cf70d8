"""CPU oracle for the Moshi RQ-Transformer frame step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and shares no code with it.
"""
from .moshi_oracle import (  # noqa: F401
    ALPHA,
    Oracle,
    Session,
    causal_attention,
    cross_entropy_loss,
    delay_codes,
    joint_sequence,
    n_depth,
    rms_norm,
    rope,
    shift_stream,
    silu,
    stream_starts,
    top2_margin,
    undelay_codes,
)
from .quant import dequantize_q8, dequantized_weights, is_linear, quantize_q8  # noqa: F401,E402
from .tts_control import TtsTextControl  # noqa: F401,E402
from . import sampling  # noqa: F401,E402
