"""Split residual vector quantiser of the Mimi codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP path shares no code with it.

Sources: the walkthrough of the Moshi technical report on 139.9.1.231, sections
"量化率" and "使用分裂RVQ学习语义-声学token" (Fig. 2); the notes page "Moshi: a
Speech-Text Foundation Model for Real-Time Dialogue", section 3a:
  * Q = 8 quantisers with N_A = 2048 centroids each; an RVQ applies VQ to the
    residual of the previous quantiser;
  * the 512-dim latent is projected to 256 dims by a linear layer before the
    quantiser and back to 512 dims before decoding;
  * split RVQ: a plain VQ (the semantic codebook) and a 7-level RVQ (the
    acoustic codebooks) are applied in parallel, and their outputs are summed.

READINGS:
  * one input projection (256 x 512) feeds both branches and one output
    projection (512 x 256) maps the summed outputs back; no biases;
  * nearest means the least squared Euclidean distance; ties go to the lowest
    index. Distances are computed here in float64 as ||r - c||^2;
  * the acoustic branch starts from the projected latent itself, not from the
    semantic branch's residual (the split removes that constraint);
  * codes[:, 0] is the semantic code and codes[:, 1..7] the acoustic levels.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def nearest(r: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Index of the nearest codeword (least squared distance, lowest index on ties)
    for each row of r [M, D] in codebook [N, D]."""
    r = np.asarray(r, dtype=np.float64)
    c = np.asarray(codebook, dtype=np.float64)
    d = ((r[:, None, :] - c[None, :, :]) ** 2).sum(axis=-1)
    return np.argmin(d, axis=1)


def encode(z: np.ndarray, w_in: np.ndarray, codebooks: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """z [M, 512] -> (codes [M, Q] int32, acoustic residual [M, 256]).

    x = z W_in^T; the semantic code is the nearest codeword of x in codebook 0;
    the acoustic levels q = 1..Q-1 each take the nearest codeword of the running
    residual (starting from x) and subtract it."""
    x = np.asarray(z, dtype=np.float64) @ np.asarray(w_in, dtype=np.float64).T
    Q = codebooks.shape[0]
    codes = np.empty((x.shape[0], Q), dtype=np.int32)
    codes[:, 0] = nearest(x, codebooks[0])
    r = x.copy()
    for q in range(1, Q):
        codes[:, q] = nearest(r, codebooks[q])
        r = r - np.asarray(codebooks[q], dtype=np.float64)[codes[:, q]]
    return codes, r


def decode(codes: np.ndarray, codebooks: np.ndarray, w_out: np.ndarray) -> np.ndarray:
    """codes [M, Q] -> z_hat [M, 512]: the sum of the chosen codewords of both
    branches, projected back by W_out."""
    cb = np.asarray(codebooks, dtype=np.float64)
    y = np.zeros((codes.shape[0], cb.shape[2]))
    for q in range(cb.shape[0]):
        y += cb[q][codes[:, q]]
    return y @ np.asarray(w_out, dtype=np.float64).T
