"""ctypes binding of ``libmoshi.so`` (declared in include/moshi.h).

Argument marshalling only: every computation runs in the library's HIP kernels.
PyTorch provides the device workspace and the caller stream. The functions
``moshi_*`` mirror the C entry points one to one; ``Moshi`` bundles them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoshi.so")

MOSHI_OK = 0
MOSHI_EINVAL = -1
MOSHI_ECONTEXT = -2
MOSHI_ENOMEM = -3
MOSHI_EHIP = -4
MOSHI_ESTATE = -5
MOSHI_F32 = 0
MOSHI_BF16 = 1
MOSHI_Q8 = 2
MOSHI_DEVICE_PTRS = 1
MOSHI_TF_FILL_KV = 2
MOSHI_TF_SKIP_DEPTH = 4
MOSHI_STEP_TEXT_ONLY = 8

_ERR_NAMES = {-1: "EINVAL", -2: "ECONTEXT", -3: "ENOMEM", -4: "EHIP", -5: "ESTATE"}


class MoshiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


class moshi_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("d_t", "n_layers_t", "n_heads_t", "ffn_t", "ctx_max",
                                               "d_d", "n_layers_d", "n_heads_d", "ffn_d",
                                               "vocab_text", "codebook", "n_q", "delay")] + \
               [("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float)] + \
               [(n, ctypes.c_int32) for n in ("dtype", "max_batch", "page_frames", "n_pages", "max_tf_tokens",
                                              "text_delay", "tts_max_tokens", "n_depth")]


class moshi_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("on_device", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class moshi_loss(ctypes.Structure):
    _fields_ = [("ce_text", ctypes.c_double), ("ce_audio", ctypes.c_double), ("ce_total", ctypes.c_double),
                ("ce_per_cb", ctypes.c_double * 8), ("n_text", ctypes.c_int64), ("n_audio", ctypes.c_int64)]


EXPORTS = (
    "moshi_workspace_bytes", "moshi_check_config", "moshi_create", "moshi_init_weights", "moshi_reset",
    "moshi_step", "moshi_forward_teacher_forced", "moshi_sync", "moshi_position", "moshi_delay_codes",
    "moshi_undelay_codes", "moshi_last_error", "moshi_destroy", "moshi_time_kernel", "moshi_read_q8",
    "moshi_tts_text", "moshi_set_sampling", "moshi_rvq_work_bytes", "moshi_rvq_encode", "moshi_rvq_decode",
    "moshi_mimi_transformer_work_bytes", "moshi_mimi_transformer", "moshi_seanet_work_bytes", "moshi_seanet_encode",
    "moshi_seanet_decode",
)
KERNELS = {"qkv": 0, "wo": 1, "ffn_gate_up": 2, "ffn_down": 3, "text_head": 4, "attn": 5, "tf_gate_up": 6,
           "tf_attn": 7}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m full_duplex_speech_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
    L.moshi_workspace_bytes.argtypes = [P(moshi_config)]
    L.moshi_workspace_bytes.restype = ctypes.c_size_t
    L.moshi_check_config.argtypes = [P(moshi_config), ctypes.c_char_p, ctypes.c_size_t]
    L.moshi_create.argtypes = [P(moshi_config), VP, VP, ctypes.c_size_t, P(VP)]
    L.moshi_init_weights.argtypes = [VP, P(moshi_tensor), ctypes.c_int]
    L.moshi_reset.argtypes = [VP, ctypes.c_int]
    L.moshi_step.argtypes = [VP, I32, VP, VP, VP, VP, VP, I32]
    L.moshi_forward_teacher_forced.argtypes = [VP, VP, I32, I32, I32, VP, VP, P(moshi_loss)]
    L.moshi_sync.argtypes = [VP]
    L.moshi_position.argtypes = [VP, ctypes.c_int]
    L.moshi_delay_codes.argtypes = [VP, I32, I32, I32, VP]
    L.moshi_undelay_codes.argtypes = [VP, I32, I32, VP]
    L.moshi_last_error.argtypes = [VP]
    L.moshi_last_error.restype = ctypes.c_char_p
    L.moshi_time_kernel.argtypes = [VP, I32, I32, I32, P(ctypes.c_float), P(ctypes.c_double)]
    L.moshi_read_q8.argtypes = [VP, ctypes.c_char_p, VP, VP, VP]
    L.moshi_tts_text.argtypes = [VP, I32, VP, VP, I32, I32, I32, ctypes.c_float, ctypes.c_float]
    L.moshi_set_sampling.argtypes = [VP, ctypes.c_float, ctypes.c_float, ctypes.c_uint64]
    L.moshi_rvq_work_bytes.argtypes = [I32, I32, I32, I32]
    L.moshi_rvq_work_bytes.restype = ctypes.c_size_t
    L.moshi_rvq_encode.argtypes = [VP, I32, I32, VP, I32, VP, I32, I32, VP, VP, VP]
    L.moshi_rvq_decode.argtypes = [VP, I32, VP, I32, I32, I32, VP, I32, VP, VP, VP]
    L.moshi_mimi_transformer_work_bytes.argtypes = [I32, I32]
    L.moshi_mimi_transformer_work_bytes.restype = ctypes.c_size_t
    L.moshi_mimi_transformer.argtypes = [VP, I32, I32, VP, I32, I32, VP, VP]
    L.moshi_seanet_work_bytes.argtypes = [I32, I32]
    L.moshi_seanet_work_bytes.restype = ctypes.c_size_t
    L.moshi_seanet_encode.argtypes = [VP, I32, I32, VP, VP, VP, VP]
    L.moshi_seanet_decode.argtypes = [VP, I32, I32, VP, VP, VP, VP]
    L.moshi_destroy.argtypes = [VP]
    L.moshi_destroy.restype = None
    for n in ("moshi_check_config", "moshi_create", "moshi_init_weights", "moshi_reset", "moshi_step",
              "moshi_forward_teacher_forced", "moshi_sync", "moshi_position", "moshi_delay_codes",
              "moshi_undelay_codes", "moshi_time_kernel", "moshi_read_q8", "moshi_tts_text",
              "moshi_set_sampling", "moshi_rvq_encode", "moshi_rvq_decode",
              "moshi_mimi_transformer", "moshi_seanet_encode", "moshi_seanet_decode"):
        getattr(L, n).restype = ctypes.c_int
    _lib = L
    return L


def _ptr(x):
    """Host numpy array or device torch tensor -> address (None stays None)."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("arrays must be C-contiguous")
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous")
        return x.data_ptr()
    raise TypeError(f"unsupported buffer type {type(x)}")


def _check(ctx, rc: int):
    if rc < 0:
        raise MoshiError(rc, lib().moshi_last_error(ctx).decode())
    return rc


def config_struct(cfg, max_batch: Optional[int] = None, page_frames: int = 64, n_pages: int = 0,
                  max_tf_tokens: int = 0, tts_max_tokens: int = 0) -> moshi_config:
    """Fill the C config from any object with the model's shape attributes."""
    c = moshi_config()
    for n in ("d_t", "n_layers_t", "n_heads_t", "ffn_t", "ctx_max", "d_d", "n_layers_d", "n_heads_d", "ffn_d",
              "vocab_text", "codebook", "n_q", "delay"):
        setattr(c, n, int(getattr(cfg, n)))
    c.rope_base = float(cfg.rope_base)
    c.norm_eps = float(cfg.norm_eps)
    c.dtype = {"bf16": MOSHI_BF16, "q8": MOSHI_Q8}.get(cfg.dtype, MOSHI_F32)
    c.max_batch = int(max_batch if max_batch is not None else cfg.batch)
    c.page_frames = page_frames
    c.n_pages = n_pages
    c.max_tf_tokens = max_tf_tokens
    c.text_delay = int(getattr(cfg, "text_delay", 0))
    c.tts_max_tokens = tts_max_tokens
    c.n_depth = int(getattr(cfg, "n_depth", 8))
    return c


# ---- one-to-one wrappers of the C entry points ---------------------------------

def moshi_workspace_bytes(c: moshi_config) -> int:
    return int(lib().moshi_workspace_bytes(ctypes.byref(c)))


def moshi_check_config(c: moshi_config) -> Tuple[int, str]:
    buf = ctypes.create_string_buffer(256)
    rc = lib().moshi_check_config(ctypes.byref(c), buf, 256)
    return rc, buf.value.decode()


def moshi_create(c: moshi_config, hip_stream: int, workspace: int, ws_bytes: int) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    rc = lib().moshi_create(ctypes.byref(c), hip_stream or None, workspace, ws_bytes, ctypes.byref(out))
    _check(None, rc)
    return out


def moshi_init_weights(ctx, tensors: Iterable[Tuple[str, object]]) -> None:
    items = list(tensors)
    arr = (moshi_tensor * len(items))()
    keep = []
    for i, (name, a) in enumerate(items):
        on_dev = not isinstance(a, np.ndarray)
        if not on_dev:
            a = np.ascontiguousarray(a, dtype=np.float32)
        keep.append(a)
        nb = name.encode()
        keep.append(nb)
        arr[i].name = nb
        arr[i].data = _ptr(a)
        arr[i].numel = int(a.size if not on_dev else a.numel())
        arr[i].on_device = 1 if on_dev else 0
    _check(ctx, lib().moshi_init_weights(ctx, arr, len(items)))


def moshi_reset(ctx, b: int = -1) -> None:
    _check(ctx, lib().moshi_reset(ctx, b))


def moshi_step(ctx, batch, user_codes, force, out_tokens, out_text_logits=None, out_audio_logits=None,
               flags: int = 0) -> None:
    _check(ctx, lib().moshi_step(ctx, batch, _ptr(user_codes), _ptr(force), _ptr(out_tokens),
                                 _ptr(out_text_logits), _ptr(out_audio_logits), flags))


def moshi_forward_teacher_forced(ctx, tokens, B, S, flags=0, text_logits=None, audio_logits=None,
                                 loss: Optional[moshi_loss] = None) -> None:
    _check(ctx, lib().moshi_forward_teacher_forced(ctx, _ptr(tokens), B, S, flags, _ptr(text_logits),
                                                   _ptr(audio_logits), ctypes.byref(loss) if loss is not None else None))


def moshi_sync(ctx) -> None:
    _check(ctx, lib().moshi_sync(ctx))


def moshi_position(ctx, b: int) -> int:
    return _check(ctx, lib().moshi_position(ctx, b))


def moshi_delay_codes(frames: np.ndarray, tau: int, pad: int) -> np.ndarray:
    f = np.ascontiguousarray(frames, dtype=np.int32)
    out = np.empty_like(f)
    _check(None, lib().moshi_delay_codes(_ptr(f), f.shape[0], tau, pad, _ptr(out)))
    return out


def moshi_undelay_codes(model: np.ndarray, tau: int) -> np.ndarray:
    m = np.ascontiguousarray(model, dtype=np.int32)
    out = np.empty((max(m.shape[0] - tau, 0), 8), dtype=np.int32)
    _check(None, lib().moshi_undelay_codes(_ptr(m), m.shape[0], tau, _ptr(out) if out.size else None))
    return out


def moshi_time_kernel(ctx, kernel: str, batch: int, iters: int) -> Tuple[float, float]:
    """(mean microseconds per launch, algorithmic work per launch) of one kernel: bytes for the frame
    kernels, floating-point operations for the teacher-forced ones ("tf_gate_up", "tf_attn")."""
    us = ctypes.c_float()
    nbytes = ctypes.c_double()
    _check(ctx, lib().moshi_time_kernel(ctx, KERNELS[kernel], batch, iters, ctypes.byref(us), ctypes.byref(nbytes)))
    return float(us.value), float(nbytes.value)


def moshi_read_q8(ctx, name: str, rows: int, cols: int):
    """(codes uint8 [rows, cols], scale float16 [rows, cols/32], min float16 [rows, cols/32]) of an
    8-bit model's linear tensor, as stored on the device."""
    codes = np.empty((rows, cols), dtype=np.uint8)
    scale = np.empty((rows, cols // 32), dtype=np.uint16)
    mn = np.empty((rows, cols // 32), dtype=np.uint16)
    _check(ctx, lib().moshi_read_q8(ctx, name.encode(), codes.ctypes.data, scale.ctypes.data, mn.ctypes.data))
    return codes, scale.view(np.float16), mn.view(np.float16)


def moshi_tts_text(ctx, conv: int, words, pad_id: int, epad_id: int, target_pad_ratio: float, bonus: float) -> None:
    """Zero-shot TTS text control of conversation ``conv``: ``words`` is a list of
    token-id lists in speaking order (an empty list switches the control off)."""
    toks = np.ascontiguousarray([t for w in words for t in w], dtype=np.int32)
    lens = np.ascontiguousarray([len(w) for w in words], dtype=np.int32)
    _check(ctx, lib().moshi_tts_text(ctx, conv, toks.ctypes.data if toks.size else None,
                                     lens.ctypes.data if lens.size else None, int(lens.size), pad_id, epad_id,
                                     target_pad_ratio, bonus))


def moshi_set_sampling(ctx, temp_text: float, temp_audio: float, seed: int) -> None:
    _check(ctx, lib().moshi_set_sampling(ctx, temp_text, temp_audio, seed))


def moshi_rvq_work_bytes(M: int, dq: int, Q: int, N: int) -> int:
    return int(lib().moshi_rvq_work_bytes(M, dq, Q, N))


def moshi_rvq_encode(z, M, dz, w_in, dq, codebooks, Q, N, codes, work, hip_stream=None) -> None:
    rc = lib().moshi_rvq_encode(_ptr(z), M, dz, _ptr(w_in), dq, _ptr(codebooks), Q, N, _ptr(codes), _ptr(work),
                                hip_stream)
    if rc:
        raise MoshiError(rc, "moshi_rvq_encode failed")


def moshi_rvq_decode(codes, M, codebooks, Q, N, dq, w_out, dz, z_hat, work, hip_stream=None) -> None:
    rc = lib().moshi_rvq_decode(_ptr(codes), M, _ptr(codebooks), Q, N, dq, _ptr(w_out), dz, _ptr(z_hat), _ptr(work),
                                hip_stream)
    if rc:
        raise MoshiError(rc, "moshi_rvq_decode failed")


def moshi_mimi_transformer_work_bytes(B: int, S: int) -> int:
    return int(lib().moshi_mimi_transformer_work_bytes(B, S))


def moshi_mimi_transformer(x, B, S, weights, n_layers, window, work, hip_stream=None) -> None:
    rc = lib().moshi_mimi_transformer(_ptr(x), B, S, _ptr(weights), n_layers, window, _ptr(work), hip_stream)
    if rc:
        raise MoshiError(rc, "moshi_mimi_transformer failed")


def moshi_seanet_work_bytes(B: int, S: int) -> int:
    return int(lib().moshi_seanet_work_bytes(B, S))


def moshi_seanet_encode(audio, B, S, weights, latents, work, hip_stream=None) -> None:
    rc = lib().moshi_seanet_encode(_ptr(audio), B, S, _ptr(weights), _ptr(latents), _ptr(work), hip_stream)
    if rc:
        raise MoshiError(rc, "moshi_seanet_encode failed")


def moshi_seanet_decode(latents, B, S, weights, audio, work, hip_stream=None) -> None:
    rc = lib().moshi_seanet_decode(_ptr(latents), B, S, _ptr(weights), _ptr(audio), _ptr(work), hip_stream)
    if rc:
        raise MoshiError(rc, "moshi_seanet_decode failed")


def moshi_last_error(ctx) -> str:
    return lib().moshi_last_error(ctx).decode()


def moshi_destroy(ctx) -> None:
    lib().moshi_destroy(ctx)


# ---- convenience object ---------------------------------------------------------

class Moshi:
    """One context with a torch-allocated workspace on the current GPU."""

    def __init__(self, cfg, max_batch: Optional[int] = None, page_frames: int = 64, n_pages: int = 0,
                 max_tf_tokens: int = 0, device: Optional[int] = None, tts_max_tokens: int = 0):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("the HIP library needs a GPU; none is visible")
        if device is not None:
            torch.cuda.set_device(device)
        self.cfg = cfg
        self.c = config_struct(cfg, max_batch, page_frames, n_pages, max_tf_tokens, tts_max_tokens)
        rc, msg = moshi_check_config(self.c)
        if rc:
            raise MoshiError(rc, msg)
        self.ws_bytes = moshi_workspace_bytes(self.c)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream().cuda_stream
        self.ctx = moshi_create(self.c, self.stream, self.ws.data_ptr(), self.ws_bytes)

    def close(self):
        if getattr(self, "ctx", None) is not None:
            moshi_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_weights(self, weights) -> None:
        items = weights.items() if isinstance(weights, dict) else weights
        moshi_init_weights(self.ctx, items)

    def reset(self, b: int = -1) -> None:
        moshi_reset(self.ctx, b)

    def position(self, b: int = 0) -> int:
        return moshi_position(self.ctx, b)

    def step(self, user_codes: np.ndarray, force: Optional[np.ndarray] = None, logits: bool = False,
             text_only: bool = False):
        """Host-pointer step: returns (tokens [B, 9] or [B, 17] with a 16-index depth,
        text_logits, audio_logits). ``force`` entries of -1 leave a slot to the model;
        ``text_only`` skips the depth; ``user_codes`` may be an int B (no user input:
        a 16-index depth draws the user's codes)."""
        cfg = self.cfg
        nd = 16 if getattr(cfg, "n_depth", 8) == 16 else 8
        if isinstance(user_codes, (int, np.integer)):
            u, B = None, int(user_codes)
        else:
            u = np.ascontiguousarray(user_codes, dtype=np.int32).reshape(-1, 8)
            B = u.shape[0]
        f = None if force is None else np.ascontiguousarray(force, dtype=np.int32).reshape(B, 9)
        tok = np.empty((B, 17 if nd == 16 else 9), dtype=np.int32)
        lt = np.empty((B, cfg.vocab_text), dtype=np.float32) if logits else None
        la = np.empty((B, nd, cfg.codebook), dtype=np.float32) if logits and not text_only else None
        moshi_step(self.ctx, B, u, f, tok, lt, la, MOSHI_STEP_TEXT_ONLY if text_only else 0)
        return tok, lt, la

    def set_sampling(self, temp_text: float, temp_audio: float, seed: int) -> None:
        moshi_set_sampling(self.ctx, temp_text, temp_audio, seed)

    def tts_text(self, words, pad_id: int, epad_id: int, target_pad_ratio: float, bonus: float, conv: int = 0):
        moshi_tts_text(self.ctx, conv, words, pad_id, epad_id, target_pad_ratio, bonus)

    def forward_teacher_forced(self, tokens: np.ndarray, fill_kv: bool = False, skip_depth: bool = False,
                               logits: bool = True, loss: bool = True):
        """Host-pointer teacher-forced pass over tokens [B, S, 17]."""
        cfg = self.cfg
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        B, S = t.shape[:2]
        flags = (MOSHI_TF_FILL_KV if fill_kv else 0) | (MOSHI_TF_SKIP_DEPTH if skip_depth else 0)
        lt = np.empty((B, S, cfg.vocab_text), dtype=np.float32) if logits else None
        la = np.empty((B, S, cfg.n_q, cfg.codebook), dtype=np.float32) if logits and not skip_depth else None
        ls = moshi_loss() if loss else None
        moshi_forward_teacher_forced(self.ctx, t, B, S, flags, lt, la, ls)
        out = None
        if ls is not None:
            out = {"ce_text": ls.ce_text, "ce_audio": ls.ce_audio, "ce_total": ls.ce_total,
                   "ce_per_cb": list(ls.ce_per_cb), "n_text": ls.n_text, "n_audio": ls.n_audio}
        return lt, la, out
