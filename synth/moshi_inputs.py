"""Model shapes, seeded random weights and seeded random token streams.

Shapes follow the configurations of the RQ-Transformer frame step studied here:
a Helium-style Temporal Transformer over time and a Depth Transformer over the
codebooks of one frame (paper walkthrough on 139.9.1.231, section
"使用 RQ-Transformer 的分层自回归建模", Fig. 3; notes page "Moshi: a Speech-Text
Foundation Model for Real-Time Dialogue", sections 3b and 3c).

Random-number recipe (identical for every consumer):
  * weight tensor number ``i`` in ``weight_specs(cfg)`` order is
    ``default_rng([seed, i]).standard_normal(shape, float32) * std``, laid out
    C-order as [out_features, in_features] for linear maps and [rows, dim] for
    embedding tables; RMSNorm gains are exactly 1.
  * linear maps use std 0.02, embedding tables (pad rows included) std 1.
  * for bf16 models every weight is rounded to the nearest bfloat16 value
    (ties to even) and handed out as float32 holding that value, so the inputs
    of both implementations are the same numbers.
  * raw token streams of conversation ``b``: stream 1 is the text stream
    (ids in [0, vocab_text)), stream 2 Moshi's 8 codebooks, stream 3 the user's
    8 codebooks (ids in [0, codebook)); stream ``k`` is drawn from
    ``default_rng([seed, 1000 + b, k]).integers(0, n, size, int32)``. These
    are codec-order frames; placing them into the delayed joint sequence is
    model arithmetic and is not done here.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Callable, Dict, Iterable, List, Optional, Tuple

import numpy as np

LINEAR_STD = 0.02
EMBED_STD = 1.0


@dataclasses.dataclass(frozen=True)
class MoshiConfig:
    name: str
    # Temporal Transformer
    d_t: int
    n_layers_t: int
    n_heads_t: int
    ffn_t: int
    ctx_max: int
    # Depth Transformer (one weight set per codebook index)
    d_d: int
    n_layers_d: int
    n_heads_d: int
    ffn_d: int
    vocab_text: int
    codebook: int = 2048
    n_q: int = 8
    delay: int = 1
    text_delay: int = 0  # > 0: text lags the audio by that many frames (ASR); < 0: audio lags text (TTS)
    rope_base: float = 10000.0
    norm_eps: float = 1e-5
    dtype: str = "f32"  # weight precision: "f32", "bf16" or "q8" (8-bit blocks of the bf16 values)
    # workload
    batch: int = 1
    prompt_frames: int = 0
    gen_frames: int = 0
    tf_batch: int = 0
    tf_frames: int = 0
    mode: str = "dialogue"  # streaming workload: "dialogue", "asr" (audio forced, text only) or "tts"
    n_depth: int = 8  # depth indices: 8 (Moshi's codebooks) or 16 (also the user's, simulated dialogues)
    temp_text: float = 0.0   # sampling temperatures of the own tokens (0 = greedy)
    temp_audio: float = 0.0

    @property
    def n_streams(self) -> int:
        return 2 * self.n_q + 1

    @property
    def pad_text(self) -> int:
        return self.vocab_text

    @property
    def pad_audio(self) -> int:
        return self.codebook

    def replace(self, **kw) -> "MoshiConfig":
        return dataclasses.replace(self, **kw)


_DEPTH_7B = dict(d_d=1024, n_layers_d=6, n_heads_d=16, ffn_d=2816)
_TEMPORAL_7B = dict(d_t=4096, n_layers_t=32, n_heads_t=32, ffn_t=11008, ctx_max=4096)

CONFIGS: Dict[str, MoshiConfig] = {
    # 50 frames (4 s at 12.5 Hz), batch 1, everything float32
    "tiny": MoshiConfig(
        name="tiny", d_t=256, n_layers_t=2, n_heads_t=4, ffn_t=688, ctx_max=64,
        d_d=128, n_layers_d=2, n_heads_d=4, ffn_d=352, vocab_text=1000,
        dtype="f32", batch=1, prompt_frames=0, gen_frames=50),
    # 375-frame prompt then 125 generated frames, float32 and bf16 weights
    "mid_f32": MoshiConfig(
        name="mid_f32", d_t=1024, n_layers_t=8, n_heads_t=16, ffn_t=2816, ctx_max=4096,
        vocab_text=32000, dtype="f32", batch=1, prompt_frames=375, gen_frames=125,
        **_DEPTH_7B),
    "mid_bf16": MoshiConfig(
        name="mid_bf16", d_t=1024, n_layers_t=8, n_heads_t=16, ffn_t=2816, ctx_max=4096,
        vocab_text=32000, dtype="bf16", batch=1, prompt_frames=375, gen_frames=125,
        **_DEPTH_7B),
    # 7B shape, batch 1: 375-frame prompt then 250 greedy frames
    "b1_7b": MoshiConfig(
        name="b1_7b", vocab_text=32000, dtype="bf16", batch=1, prompt_frames=375,
        gen_frames=250, **_TEMPORAL_7B, **_DEPTH_7B),
    # the same model with its linear maps in 8-bit blocks (quantised from the bf16 values)
    "mid_q8": MoshiConfig(
        name="mid_q8", d_t=1024, n_layers_t=8, n_heads_t=16, ffn_t=2816, ctx_max=4096,
        vocab_text=32000, dtype="q8", batch=1, prompt_frames=375, gen_frames=125,
        **_DEPTH_7B),
    "b1_7b_q8": MoshiConfig(
        name="b1_7b_q8", vocab_text=32000, dtype="q8", batch=1, prompt_frames=375,
        gen_frames=250, **_TEMPORAL_7B, **_DEPTH_7B),
    # simulated dialogues: the depth also predicts the user's 8 codebooks
    "tiny_sim": MoshiConfig(
        name="tiny_sim", d_t=256, n_layers_t=2, n_heads_t=4, ffn_t=688, ctx_max=64,
        d_d=128, n_layers_d=2, n_heads_d=4, ffn_d=352, vocab_text=1000, n_depth=16,
        dtype="f32", batch=1, prompt_frames=0, gen_frames=40),
    "mid_sim": MoshiConfig(
        name="mid_sim", d_t=1024, n_layers_t=8, n_heads_t=16, ffn_t=2816, ctx_max=4096,
        vocab_text=32000, n_depth=16, dtype="bf16", batch=1, prompt_frames=0, gen_frames=40,
        **_DEPTH_7B),
    "b1_7b_sim": MoshiConfig(
        name="b1_7b_sim", vocab_text=32000, dtype="bf16", batch=1, prompt_frames=375,
        gen_frames=250, n_depth=16, temp_text=0.7, temp_audio=0.8, **_TEMPORAL_7B, **_DEPTH_7B),
    # the batch-1 workload with temperature sampling (text 0.7, audio 0.8)
    "b1_7b_sampled": MoshiConfig(
        name="b1_7b_sampled", vocab_text=32000, dtype="bf16", batch=1, prompt_frames=375,
        gen_frames=250, temp_text=0.7, temp_audio=0.8, **_TEMPORAL_7B, **_DEPTH_7B),
    # streaming ASR and TTS: text and audio 2 s (25 frames) apart, acoustic delay 2
    "tiny_asr": MoshiConfig(
        name="tiny_asr", d_t=256, n_layers_t=2, n_heads_t=4, ffn_t=688, ctx_max=64,
        d_d=128, n_layers_d=2, n_heads_d=4, ffn_d=352, vocab_text=1000, delay=2, text_delay=25,
        dtype="f32", batch=1, prompt_frames=0, gen_frames=50, mode="asr"),
    "tiny_tts": MoshiConfig(
        name="tiny_tts", d_t=256, n_layers_t=2, n_heads_t=4, ffn_t=688, ctx_max=64,
        d_d=128, n_layers_d=2, n_heads_d=4, ffn_d=352, vocab_text=1000, delay=2, text_delay=-25,
        dtype="f32", batch=1, prompt_frames=0, gen_frames=50, mode="tts"),
    "mid_asr": MoshiConfig(
        name="mid_asr", d_t=1024, n_layers_t=8, n_heads_t=16, ffn_t=2816, ctx_max=4096,
        vocab_text=32000, delay=2, text_delay=25, dtype="bf16", batch=1, prompt_frames=0,
        gen_frames=100, mode="asr", **_DEPTH_7B),
    "mid_tts": MoshiConfig(
        name="mid_tts", d_t=1024, n_layers_t=8, n_heads_t=16, ffn_t=2816, ctx_max=4096,
        vocab_text=32000, delay=2, text_delay=-25, dtype="bf16", batch=1, prompt_frames=0,
        gen_frames=100, mode="tts", **_DEPTH_7B),
    "b1_7b_asr": MoshiConfig(
        name="b1_7b_asr", vocab_text=32000, delay=2, text_delay=25, dtype="bf16", batch=1,
        prompt_frames=375, gen_frames=250, mode="asr", **_TEMPORAL_7B, **_DEPTH_7B),
    "b1_7b_tts": MoshiConfig(
        name="b1_7b_tts", vocab_text=32000, delay=2, text_delay=-25, dtype="bf16", batch=1,
        prompt_frames=375, gen_frames=250, mode="tts", **_TEMPORAL_7B, **_DEPTH_7B),
    # 7B shape, 8 conversations at 5-minute context
    "b8_7b_5min": MoshiConfig(
        name="b8_7b_5min", vocab_text=32000, dtype="bf16", batch=8, prompt_frames=3750,
        gen_frames=125, **_TEMPORAL_7B, **_DEPTH_7B),
    # 7B shape, teacher-forced scoring of 4 x 3750 frames
    "tf_7b": MoshiConfig(
        name="tf_7b", vocab_text=32000, dtype="bf16", batch=4, tf_batch=4, tf_frames=3750,
        **_TEMPORAL_7B, **_DEPTH_7B),
}


def config(preset: str, **overrides) -> MoshiConfig:
    cfg = CONFIGS[preset]
    return cfg.replace(**overrides) if overrides else cfg


def weight_specs(cfg: MoshiConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Ordered list of (name, shape, init) with init in {"linear", "embed", "ones"}."""
    d, F, Vt, NA = cfg.d_t, cfg.ffn_t, cfg.vocab_text, cfg.codebook
    dd, Fd = cfg.d_d, cfg.ffn_d
    specs: List[Tuple[str, Tuple[int, ...], str]] = []
    # one input table per sub-stream: 0 = text, 1..8 Moshi codebooks, 9..16 user codebooks
    for k in range(cfg.n_streams):
        rows = (Vt if k == 0 else NA) + 1  # + pad row
        specs.append((f"temporal.emb.{k}", (rows, d), "embed"))
    for l in range(cfg.n_layers_t):
        p = f"temporal.layers.{l}."
        specs += [
            (p + "attn_norm", (d,), "ones"),
            (p + "wq", (d, d), "linear"),
            (p + "wk", (d, d), "linear"),
            (p + "wv", (d, d), "linear"),
            (p + "wo", (d, d), "linear"),
            (p + "ffn_norm", (d,), "ones"),
            (p + "w_gate", (F, d), "linear"),
            (p + "w_up", (F, d), "linear"),
            (p + "w_down", (d, F), "linear"),
        ]
    specs += [("temporal.out_norm", (d,), "ones"), ("temporal.text_head", (Vt, d), "linear")]
    for j in range(cfg.n_depth):
        p = f"depth.{j}."
        rows = (Vt if j == 0 else NA) + 1
        specs += [(p + "in_proj", (dd, d), "linear"), (p + "emb", (rows, dd), "embed")]
        for l in range(cfg.n_layers_d):
            q = p + f"layers.{l}."
            specs += [
                (q + "attn_norm", (dd,), "ones"),
                (q + "wq", (dd, dd), "linear"),
                (q + "wk", (dd, dd), "linear"),
                (q + "wv", (dd, dd), "linear"),
                (q + "wo", (dd, dd), "linear"),
                (q + "ffn_norm", (dd,), "ones"),
                (q + "w_gate", (Fd, dd), "linear"),
                (q + "w_up", (Fd, dd), "linear"),
                (q + "w_down", (dd, Fd), "linear"),
            ]
        specs += [(p + "out_norm", (dd,), "ones"), (p + "head", (NA, dd), "linear")]
    return specs


def param_count(cfg: MoshiConfig) -> int:
    return int(sum(int(np.prod(s)) for _, s, _ in weight_specs(cfg)))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place; returns ``a``."""
    assert a.dtype == np.float32
    u = a.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return a


def generate_weight(cfg: MoshiConfig, ordinal: int, seed: int = 0) -> np.ndarray:
    name, shape, init = weight_specs(cfg)[ordinal]
    return _draw(shape, init, seed, ordinal, cfg.dtype)


def _draw(shape, init, seed, ordinal, dtype) -> np.ndarray:
    if init == "ones":
        return np.ones(shape, dtype=np.float32)
    a = np.random.default_rng([seed, ordinal]).standard_normal(shape, dtype=np.float32)
    a *= np.float32(LINEAR_STD if init == "linear" else EMBED_STD)
    if dtype in ("bf16", "q8"):
        bf16_round(a)
    return a


def generate_weights(cfg: MoshiConfig, seed: int = 0, threads: Optional[int] = None,
                     sink: Optional[Callable[[str, np.ndarray], None]] = None,
                     keep: bool = True) -> Dict[str, np.ndarray]:
    """Draw every weight tensor. With ``sink``, each tensor is passed to it as soon as it
    is drawn (``sink`` runs on the calling thread, in spec order); with ``keep=False``
    tensors are dropped after ``sink`` saw them, which bounds host memory for 7B shapes."""
    specs = weight_specs(cfg)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    out: Dict[str, np.ndarray] = {}

    def job(i):
        name, shape, init = specs[i]
        return name, _draw(shape, init, seed, i, cfg.dtype)

    if threads <= 1:
        for i in range(len(specs)):
            name, a = job(i)
            if sink is not None:
                sink(name, a)
            if keep:
                out[name] = a
        return out
    with _cf.ThreadPoolExecutor(threads) as ex:
        # bounded look-ahead so that keep=False streams with O(threads) tensors alive
        window = 2 * threads
        futs = {}
        nxt = 0
        for i in range(len(specs)):
            while nxt < len(specs) and nxt < i + window:
                futs[nxt] = ex.submit(job, nxt)
                nxt += 1
            name, a = futs.pop(i).result()
            if sink is not None:
                sink(name, a)
            if keep:
                out[name] = a
    return out


def raw_frames(cfg: MoshiConfig, b: int, n_frames: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """Codec-order random frames of conversation ``b``: text [T], moshi [T, n_q], user [T, n_q]."""
    def draw(stream, n, shape):
        return np.random.default_rng([seed, 1000 + b, stream]).integers(0, n, size=shape, dtype=np.int32)
    return {
        "text": draw(1, cfg.vocab_text, (n_frames,)),
        "moshi": draw(2, cfg.codebook, (n_frames, cfg.n_q)),
        "user": draw(3, cfg.codebook, (n_frames, cfg.n_q)),
    }
