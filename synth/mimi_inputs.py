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
