"""Pins of the oracle's 8-bit block weight format (block-32 asymmetric MinMax,
float16 scale and min): values placed exactly on a block grid round-trip
unchanged, every code 0..255 is reachable, the dequantisation error of a
random block is at most half a step plus the float16 rounding of the stored
minimum, constant blocks store scale 0, and the codes are monotone in the
weights."""
import numpy as np
import pytest

from oracle.quant import dequantize_q8, dequantized_weights, is_linear, quantize_q8


def test_grid_values_round_trip_exactly():
    # min and scale exactly representable in float16 and float32 arithmetic exact:
    # w = m + q * s for q = 0..255 in shuffled order, two rows, four blocks
    rng = np.random.default_rng(3)
    m, s = np.float32(-0.75), np.float32(2.0 ** -9)
    # every block holds both ends, so its range is exactly 255 steps
    blocks = []
    for b in range(8):
        qb = rng.integers(0, 256, 32)
        qb[0], qb[1] = 0, 255
        blocks.append(qb)
    qq = np.stack(blocks).reshape(2, 128)
    w = (m + qq.astype(np.float32) * s).astype(np.float32)
    qz, sc, mn = quantize_q8(w)
    assert np.all(sc.astype(np.float32) == s) and np.all(mn.astype(np.float32) == m)
    assert np.array_equal(qz.astype(np.int64), qq)
    assert np.array_equal(dequantize_q8(qz, sc, mn), w)


def test_random_block_error_bound_and_monotone():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    q, sc, mn = quantize_q8(w)
    d = dequantize_q8(q, sc, mn)
    b = w.reshape(64, 8, 32)
    step = sc.astype(np.float64)[..., None]
    # |w - w'| <= step/2 + |min - min16| + float32 rounding
    dmin = np.abs(b.min(-1) - mn.astype(np.float64))[..., None]
    err = np.abs(d.reshape(64, 8, 32).astype(np.float64) - b)
    assert np.all(err <= step * 0.5 + dmin + 1e-7)
    assert err.max() > 0.1 * step.max()  # not a degenerate identity
    # monotone codes inside each block
    for r in range(4):
        for k in range(8):
            o = np.argsort(b[r, k], kind="stable")
            assert np.all(np.diff(q.reshape(64, 8, 32)[r, k][o].astype(int)) >= 0)
    assert q.min() == 0 and q.max() == 255


def test_constant_block_and_bytes():
    w = np.full((1, 64), 0.125, dtype=np.float32)
    w[0, 32:] = -3.0
    q, sc, mn = quantize_q8(w)
    assert np.all(q == 0) and np.all(sc == 0)
    assert np.array_equal(dequantize_q8(q, sc, mn), w)
    # storage: one byte per weight plus two float16 values per 32 weights
    assert q.nbytes + sc.nbytes + mn.nbytes == 64 * 1.125


def test_linear_map_selection():
    for n in ("temporal.layers.3.wq", "temporal.layers.0.w_down", "temporal.text_head", "depth.2.in_proj",
              "depth.7.head", "depth.1.layers.5.w_gate"):
        assert is_linear(n)
    for n in ("temporal.emb.4", "depth.3.emb", "temporal.out_norm", "temporal.layers.1.attn_norm", "depth.0.out_norm"):
        assert not is_linear(n)
    w = {"temporal.text_head": np.ones((2, 32), np.float32) * 0.5, "temporal.emb.0": np.full((2, 32), 0.3, np.float32)}
    dq = dequantized_weights(w)
    assert np.array_equal(dq["temporal.emb.0"], w["temporal.emb.0"])
