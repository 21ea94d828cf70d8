"""8-bit block weight format of the oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP path shares no code with it.

Source: the walkthrough of the Moshi technical report on 139.9.1.231 ("论文解读"),
section "压缩Moshi及其对语音质量的影响", paragraph "量化格式": weights are quantised
asymmetrically (MinMax) in blocks, the temporal and the depth Transformer alike;
the initial embedding tables and the RMSNorms stay unquantised; activations are
quantised dynamically to 8 bits (AbsMax) at each linear input. The Table 10
caption of that section fixes the block size at 32 and the quantisation
parameters as float16. The online demo keeps 8-bit weights.

READINGS (the page gives the scheme, not its arithmetic):
  * a block is 32 consecutive weights along the input dimension of one row of a
    linear map; its 256 levels span [min, max] of the block:
        scale = (max - min) / 255,  w ~ min + q * scale,  q in 0..255;
  * scale and min are stored in float16 (round to nearest even), and q is
    chosen against the stored values: q = clip(round_half_even((w - min16) /
    scale16), 0, 255), computed in float32; a block with max == min stores
    scale 0 and q = 0;
  * the linear maps are the attention projections, the gated FFN, the text
    head, the depth input projections and the depth heads; the embedding
    tables and the RMSNorm gains stay unquantised;
  * DEVIATION, not a reading: activations stay unquantised (weight-only
    8-bit). At batch 1 the frame step is bound by the weight stream, which the
    activation scale does not shrink.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

BLOCK = 32
LINEAR_SUFFIXES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "text_head", "in_proj", "head")


def is_linear(name: str) -> bool:
    """Whether tensor ``name`` (synth naming) is a linear map stored in 8 bits."""
    return name.rsplit(".", 1)[-1] in LINEAR_SUFFIXES


def quantize_q8(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """w float32 [N, K] (K a multiple of 32) -> (q uint8 [N, K], scale float16
    [N, K/32], min float16 [N, K/32]), per the block MinMax reading above."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % BLOCK == 0
    b = w.reshape(N, K // BLOCK, BLOCK)
    mn = b.min(axis=-1)
    mx = b.max(axis=-1)
    scale16 = ((mx - mn) / np.float32(255)).astype(np.float16)
    min16 = mn.astype(np.float16)
    s = scale16.astype(np.float32)
    m = min16.astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1))
    q = np.rint((b - m[..., None]) / safe[..., None])
    q = np.where(s[..., None] > 0, q, 0)
    q = np.clip(q, 0, 255).astype(np.uint8)
    return q.reshape(N, K), scale16, min16


def dequantize_q8(q: np.ndarray, scale16: np.ndarray, min16: np.ndarray) -> np.ndarray:
    """The stored block values: min + q * scale, in float32."""
    N, K = q.shape
    s = scale16.astype(np.float32)[..., None]
    m = min16.astype(np.float32)[..., None]
    return (q.reshape(N, K // BLOCK, BLOCK).astype(np.float32) * s + m).reshape(N, K)


def dequantized_weights(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """The weights an 8-bit model computes with: every linear map replaced by its
    quantise-dequantise image, everything else unchanged."""
    out = {}
    for name, w in weights.items():
        out[name] = dequantize_q8(*quantize_q8(w)) if is_linear(name) else w
    return out
