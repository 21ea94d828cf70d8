"""Seeded random weights and latents for Mimi's bottleneck Transformer.

Recipe: tensor ``i`` of layer ``l``, in the order (ln1 gain, ln1 bias, Wq, Wk,
Wv, Wo, LayerScale 1, ln2 gain, ln2 bias, W1, W2, LayerScale 2), is drawn from
``default_rng([seed, 500 + l, i])``:
  * linear maps [out, in]: standard normal * 1/sqrt(in);
  * LayerNorm gains: 1 + 0.1 * standard normal; biases: 0.1 * standard normal;
  * LayerScale vectors: ``scale`` * (1 + 0.5 * uniform(-1, 1)) -- the pages
    initialise them at 0.01; tests use a larger scale so that every branch
    weighs on the output.
Latents of sequence ``b``: ``default_rng([seed, 900 + b]).standard_normal((S, d))``.
The packed layout (one float32 buffer, layers back to back, tensors in the order
above, each C-order) is what the library's Transformer entry point reads.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

NAMES = ("ln1_g", "ln1_b", "wq", "wk", "wv", "wo", "scale1", "ln2_g", "ln2_b", "w1", "w2", "scale2")


def shapes(d: int = 512, f: int = 2048) -> List[Tuple[int, ...]]:
    return [(d,), (d,), (d, d), (d, d), (d, d), (d, d), (d,), (d,), (d,), (f, d), (d, f), (d,)]


def mimi_weights(n_layers: int = 8, d: int = 512, f: int = 2048, seed: int = 0,
                 scale: float = 0.01) -> Dict[str, np.ndarray]:
    out = {}
    for l in range(n_layers):
        for i, (name, shp) in enumerate(zip(NAMES, shapes(d, f))):
            rng = np.random.default_rng([seed, 500 + l, i])
            if name.startswith("w"):
                v = rng.standard_normal(shp, dtype=np.float32) / np.float32(np.sqrt(shp[1]))
            elif name.endswith("_g"):
                v = 1 + 0.1 * rng.standard_normal(shp, dtype=np.float32)
            elif name.endswith("_b"):
                v = 0.1 * rng.standard_normal(shp, dtype=np.float32)
            else:
                v = scale * (1 + 0.5 * rng.uniform(-1, 1, shp)).astype(np.float32)
            out[f"mimi.layers.{l}.{name}"] = v.astype(np.float32)
    return out


def pack(weights: Dict[str, np.ndarray], n_layers: int) -> np.ndarray:
    return np.concatenate([weights[f"mimi.layers.{l}.{n}"].reshape(-1) for l in range(n_layers) for n in NAMES])


def latents(B: int, S: int, d: int = 512, seed: int = 0) -> np.ndarray:
    return np.stack([np.random.default_rng([seed, 900 + b]).standard_normal((S, d)).astype(np.float32)
                     for b in range(B)])


# ---------------------------------------------------------------------------
# SEANet encoder / decoder weights
# ---------------------------------------------------------------------------
ENC_STRIDES = (4, 5, 6, 8)


def seanet_layers(base: int = 64, dim: int = 512):
    """(name, kind, c_in, c_out, kernel, stride) of every convolution, encoder then
    decoder, in the packed order. kind: "conv" (weight [c_out][c_in][k]) or "tconv"
    (transposed, weight [c_in][c_out][k])."""
    enc = [("enc.in", "conv", 1, base, 7, 1)]
    c = base
    for i, s in enumerate(ENC_STRIDES):
        enc += [(f"enc.{i}.res_a", "conv", c, c // 2, 3, 1), (f"enc.{i}.res_b", "conv", c // 2, c, 1, 1),
                (f"enc.{i}.down", "conv", c, 2 * c, 2 * s, s)]
        c *= 2
    enc.append(("enc.out", "conv", c, dim, 4, 2))
    dec = [("dec.in", "tconv", dim, c, 4, 2)]
    for i, s in enumerate(reversed(ENC_STRIDES)):
        dec += [(f"dec.{i}.up", "tconv", c, c // 2, 2 * s, s), (f"dec.{i}.res_a", "conv", c // 2, c // 4, 3, 1),
                (f"dec.{i}.res_b", "conv", c // 4, c // 2, 1, 1)]
        c //= 2
    dec.append(("dec.out", "conv", c, 1, 7, 1))
    return enc, dec


def seanet_weights(seed: int = 0, base: int = 64, dim: int = 512) -> Dict[str, np.ndarray]:
    """Convolution weights, standard normal * 1/sqrt(c_in * k) (activations stay of
    order one), tensor ``i`` of the packed order drawn from default_rng([seed, 700 + i])."""
    enc, dec = seanet_layers(base, dim)
    out = {}
    for i, (name, kind, ci, co, k, _) in enumerate(enc + dec):
        shp = (co, ci, k) if kind == "conv" else (ci, co, k)
        rng = np.random.default_rng([seed, 700 + i])
        out[name] = (rng.standard_normal(shp, dtype=np.float32) / np.float32(np.sqrt(ci * k))).astype(np.float32)
    return out


def pack_seanet(weights: Dict[str, np.ndarray], part: str, base: int = 64, dim: int = 512) -> np.ndarray:
    enc, dec = seanet_layers(base, dim)
    layers = enc if part == "enc" else dec
    return np.concatenate([weights[n].reshape(-1) for n, *_ in layers])


def audio(B: int, n_samples: int, seed: int = 0) -> np.ndarray:
    """Seeded test signals: a sum of three random sinusoids plus 0.1 white noise."""
    out = np.empty((B, n_samples), dtype=np.float32)
    t = np.arange(n_samples) / 24000.0
    for b in range(B):
        rng = np.random.default_rng([seed, 800 + b])
        f = rng.uniform(80, 4000, 3)
        a = rng.uniform(0.1, 0.5, 3)
        x = sum(a[i] * np.sin(2 * np.pi * f[i] * t + rng.uniform(0, 6.28)) for i in range(3))
        out[b] = (x + 0.1 * rng.standard_normal(n_samples)).astype(np.float32)
    return out
