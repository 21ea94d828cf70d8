"""SEANet causal convolutional encoder and decoder of the Mimi codec -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP path shares no code with it.

Source: the walkthrough of the Moshi technical report on 139.9.1.231, section
on Mimi's baseline architecture (borrowed from SoundStream and Encodec): a
SEANet autoencoder whose encoder projects a mono 24 kHz waveform to 512-dim
latents through cascaded residual convolution blocks alternating dilated and
strided convolutions, with ELU and weight normalisation; every convolution is
causal; four blocks with strides (4, 5, 6, 8) and a final stride-2 convolution
give 12.5 frames/s; the decoder mirrors it with transposed convolutions. The
notes page section 3a repeats the strides.

READINGS (the pages give the strides and the ingredients only):
  * 64 channels after a kernel-7 input convolution, doubled by each strided
    convolution (64, 128, 256, 512, 1024), then a kernel-4 stride-2
    convolution to 512;
  * one residual unit per block, before its strided convolution:
    x + conv_k1(ELU(conv_k3(ELU(x)))), halving then restoring the channels;
  * a strided convolution has kernel 2 * stride and takes ELU of its input;
    so do the output convolutions;
  * causal padding: (k - 1) * dilation + 1 - stride zeros on the left, so a
    frame's output depends on its own and earlier samples only;
  * decoder: kernel-4 stride-2 transposed convolution 512 -> 1024, then per
    stride (8, 6, 5, 4) an ELU + transposed convolution (kernel 2 * stride,
    channels halved, the last kernel - stride outputs trimmed) and a residual
    unit; a final ELU + kernel-7 convolution to one channel;
  * no biases; weight normalisation is a parametrisation of the weights and is
    folded into them; ELU with alpha 1; dilation 1.
Arrays are channel-major [C][T]; float64.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def elu(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0, x, np.expm1(np.minimum(x, 0)))


def conv1d(x: np.ndarray, w: np.ndarray, stride: int = 1, dilation: int = 1) -> np.ndarray:
    """Causal convolution: x [C_in][T], w [C_out][C_in][K] -> [C_out][T / stride]."""
    c_in, T = x.shape
    c_out, _, K = w.shape
    pad = (K - 1) * dilation + 1 - stride
    xp = np.concatenate([np.zeros((c_in, pad)), x], axis=1)
    n = T // stride
    y = np.zeros((c_out, n))
    for k in range(K):
        y += w[:, :, k] @ xp[:, k * dilation: k * dilation + stride * n: stride]
    return y


def tconv1d(x: np.ndarray, w: np.ndarray, stride: int) -> np.ndarray:
    """Causal transposed convolution: x [C_in][T], w [C_in][C_out][K] ->
    [C_out][T * stride] (the full output's last K - stride samples trimmed)."""
    c_in, T = x.shape
    _, c_out, K = w.shape
    full = np.zeros((c_out, (T - 1) * stride + K))
    for k in range(K):
        full[:, k: k + stride * T: stride] += w[:, :, k].T @ x
    return full[:, :T * stride]


def residual(x: np.ndarray, wa: np.ndarray, wb: np.ndarray) -> np.ndarray:
    return x + conv1d(elu(conv1d(elu(x), wa)), wb)


def encode(audio: np.ndarray, w: Dict[str, np.ndarray], strides=(4, 5, 6, 8)) -> np.ndarray:
    """audio [T] (T a multiple of 1920) -> latents [T / 1920][512]."""
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    x = conv1d(np.asarray(audio, dtype=np.float64)[None, :], f["enc.in"])
    for i, s in enumerate(strides):
        x = residual(x, f[f"enc.{i}.res_a"], f[f"enc.{i}.res_b"])
        x = conv1d(elu(x), f[f"enc.{i}.down"], stride=s)
    return conv1d(elu(x), f["enc.out"], stride=2).T


def decode(latents: np.ndarray, w: Dict[str, np.ndarray], strides=(4, 5, 6, 8)) -> np.ndarray:
    """latents [S][512] -> audio [S * 1920]."""
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    x = tconv1d(np.asarray(latents, dtype=np.float64).T, f["dec.in"], 2)
    for i, s in enumerate(reversed(strides)):
        x = tconv1d(elu(x), f[f"dec.{i}.up"], s)
        x = residual(x, f[f"dec.{i}.res_a"], f[f"dec.{i}.res_b"])
    return conv1d(elu(x), f["dec.out"])[0]
