"""Bottleneck Transformer of the Mimi codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP path shares no code with it.

Sources: the walkthrough of the Moshi technical report on 139.9.1.231, section
"基于 Transformer 的瓶颈" (two Transformers, one before and one after the
quantiser: 8 layers, 8 heads, RoPE, a 250-frame (20 s) limited context, GELU,
model width 512, MLP width 2048, LayerScale initialised at 0.01, causal masks);
the notes page "Moshi: a Speech-Text Foundation Model for Real-Time Dialogue",
section 3a (the same list).

READINGS (the pages list the ingredients, not the block):
  * pre-norm residual blocks: x += g1 * Wo Attn(LN1(x)); x += g2 * W2 GELU(W1 LN2(x)),
    with g1, g2 the per-channel LayerScale vectors;
  * the norm is LayerNorm with gain and bias, epsilon 1e-5 (the pages name no
    norm; this is the standard Transformer one);
  * linear maps have no biases; GELU is the exact x * Phi(x) (erf form);
  * RoPE rotates consecutive pairs (x_2i, x_2i+1) by pos * base^(-2i/hd),
    base 10000, as in the temporal Transformer's reading;
  * the limited context is a sliding window: query t attends to keys
    max(0, t - 249) .. t;
  * positions restart at 0 for each sequence.
"""
from __future__ import annotations

from math import sqrt
from typing import Dict, List

import numpy as np
from scipy.special import erf

D_MODEL, N_HEADS, D_MLP, N_LAYERS, WINDOW = 512, 8, 2048, 8, 250


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(x: np.ndarray) -> np.ndarray:
    """x * Phi(x) = x * (1 + erf(x / sqrt 2)) / 2."""
    return x * 0.5 * (1.0 + erf(x / sqrt(2.0)))


def rope(x: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """x [S, H, hd] rotated by position (axis 0), consecutive pairs."""
    S, H, hd = x.shape
    i = np.arange(hd // 2)
    ang = np.arange(S)[:, None] * base ** (-2.0 * i / hd)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def window_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int) -> np.ndarray:
    """Per head: softmax(q k^T / sqrt(hd)) v over keys t-window+1 .. t. [S, H, hd]."""
    S, H, hd = q.shape
    out = np.empty_like(q)
    for h in range(H):
        sc = q[:, h] @ k[:, h].T / np.sqrt(hd)
        t = np.arange(S)
        allowed = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - window)
        sc = np.where(allowed, sc, -np.inf)
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h] = p @ v[:, h]
    return out


def layer_names(l: int) -> List[str]:
    p = f"mimi.layers.{l}."
    return [p + n for n in ("ln1_g", "ln1_b", "wq", "wk", "wv", "wo", "scale1", "ln2_g", "ln2_b", "w1", "w2",
                            "scale2")]


def layer_shapes(d: int = D_MODEL, f: int = D_MLP) -> List[tuple]:
    return [(d,), (d,), (d, d), (d, d), (d, d), (d, d), (d,), (d,), (d,), (f, d), (d, f), (d,)]


def forward(x: np.ndarray, weights: Dict[str, np.ndarray], n_layers: int = N_LAYERS, n_heads: int = N_HEADS,
            window: int = WINDOW) -> np.ndarray:
    """One sequence x [S, d] through the Transformer (float64)."""
    h = np.asarray(x, dtype=np.float64).copy()
    S, d = h.shape
    hd = d // n_heads
    for l in range(n_layers):
        w = {n.rsplit(".", 1)[1]: np.asarray(weights[n], dtype=np.float64) for n in layer_names(l)}
        n = layer_norm(h, w["ln1_g"], w["ln1_b"])
        q = rope((n @ w["wq"].T).reshape(S, n_heads, hd))
        k = rope((n @ w["wk"].T).reshape(S, n_heads, hd))
        v = (n @ w["wv"].T).reshape(S, n_heads, hd)
        a = window_attention(q, k, v, window).reshape(S, d)
        h = h + w["scale1"] * (a @ w["wo"].T)
        n = layer_norm(h, w["ln2_g"], w["ln2_b"])
        h = h + w["scale2"] * (gelu(n @ w["w1"].T) @ w["w2"].T)
    return h
