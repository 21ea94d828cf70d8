"""Temperature sampling with a counter-based generator -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP path shares no code with it.

Source: the walkthrough of the Moshi technical report on 139.9.1.231 samples
at temperature 0.6 for streaming TTS (the ASR/TTS metrics paragraph after
Table 9) and at 0.8 for the audio-quality samples of the quantised models
(section "压缩Moshi及其对语音质量的影响", results on audio quality).
The pages fix neither the generator nor the sampling algorithm, so this module
defines them (READINGS below); the library implements the same definitions.

READINGS:
  * a draw at temperature T > 0 from logits l picks argmax_i (l_i / T + g_i),
    with g_i = -log(-log(u_i)) standard Gumbel noise and u_i uniform on (0, 1):
    the Gumbel-max form of categorical sampling from softmax(l / T). T = 0 is
    the greedy argmax. Ties go to the lowest index;
  * u_i comes from Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC'11): key (seed, 0), counter
    (i // 4, position, conversation, slot), word i % 4 of the output. A word x
    gives u = (2 * (x >> 41) + 1) * 2^-24, exact in float32 and never 0 or 1;
  * the score l_i / T + g_i and the Gumbel transform are evaluated in float32,
    the precision of the device kernel that takes the same decision;
  * position is the 0-based position of the step, conversation the index in the
    batch, slot 0 the text and 1..8 Moshi's codebooks.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

# Philox4x64 round multipliers and key increments (the SC'11 paper's constants)
_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mul_hi_lo(a: np.ndarray, b: np.uint64):
    """Full 128-bit product of uint64 values, from 32-bit limbs: (high, low) words."""
    a_lo, a_hi = a & _LO, a >> _S32
    b_lo, b_hi = b & _LO, b >> _S32
    ll, lh, hl, hh = a_lo * b_lo, a_lo * b_hi, a_hi * b_lo, a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO) + (hl & _LO)
    lo = (ll & _LO) | ((mid & _LO) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64(counter: np.ndarray, key) -> np.ndarray:
    """Philox4x64-10 of counters [..., 4] (uint64) under key (k0, k1): 10 rounds of
    two 64x64 -> 128-bit multiplies, the key bumped by the Weyl constants between
    rounds. Returns the output words [..., 4]."""
    with np.errstate(over="ignore"):
        c = np.array(counter, dtype=np.uint64)
        c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
        k0, k1 = np.uint64(key[0]), np.uint64(key[1])
        for r in range(10):
            if r:
                k0, k1 = k0 + _W0, k1 + _W1
            hi0, lo0 = _mul_hi_lo(c0, _M0)
            hi1, lo1 = _mul_hi_lo(c2, _M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        return np.stack([c0, c1, c2, c3], axis=-1)


def uniforms(n: int, seed: int, position: int, conversation: int, slot: int) -> np.ndarray:
    """u_0..u_{n-1} (float32, open interval (0, 1)) of one draw."""
    groups = (n + 3) // 4
    ctr = np.zeros((groups, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(groups, dtype=np.uint64)
    ctr[:, 1] = position
    ctr[:, 2] = conversation
    ctr[:, 3] = slot
    x = philox4x64(ctr, (seed, 0)).reshape(-1)[:n]
    m = (x >> np.uint64(41)).astype(np.float64)
    return ((2.0 * m + 1.0) * 2.0 ** -24).astype(np.float32)


def gumbel(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.float32)
    return -np.log(-np.log(u))


def scores(logits: np.ndarray, temperature: float, u: np.ndarray) -> np.ndarray:
    """The perturbed scores l / T + g in float32."""
    l32 = np.asarray(logits, dtype=np.float32)
    return l32 / np.float32(temperature) + gumbel(u)


def sample(logits: np.ndarray, temperature: float, seed: int = 0, position: int = 0, conversation: int = 0,
           slot: int = 0, u: Optional[np.ndarray] = None) -> int:
    """One draw: greedy argmax at T = 0, else the Gumbel-max pick."""
    if temperature < 0:
        raise ValueError("temperature must be >= 0")
    if temperature == 0:
        return int(np.argmax(logits))
    if u is None:
        u = uniforms(len(logits), seed, position, conversation, slot)
    return int(np.argmax(scores(logits, temperature, u)))
