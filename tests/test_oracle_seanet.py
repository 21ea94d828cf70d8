"""Oracle pins for the SEANet encoder and decoder. All on the CPU."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from conftest import read_golden
from oracle.seanet import conv1d, decode, elu, encode, tconv1d
from synth.mimi_inputs import audio, seanet_weights


@pytest.mark.parametrize("K,stride,dil", [(7, 1, 1), (3, 1, 2), (8, 4, 1), (10, 5, 1), (4, 2, 1)])
def test_conv_matches_torch_with_left_padding(K, stride, dil):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 40))
    w = rng.standard_normal((3, 5, K))
    pad = (K - 1) * dil + 1 - stride
    ref = F.conv1d(F.pad(torch.tensor(x)[None], (pad, 0)), torch.tensor(w), stride=stride, dilation=dil)[0]
    np.testing.assert_allclose(conv1d(x, w, stride, dil), ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K,stride", [(4, 2), (16, 8), (10, 5)])
def test_tconv_matches_torch_trimmed(K, stride):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 9))
    w = rng.standard_normal((6, 4, K))
    ref = F.conv_transpose1d(torch.tensor(x)[None], torch.tensor(w), stride=stride)[0, :, :9 * stride]
    np.testing.assert_allclose(tconv1d(x, w, stride), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_elu_matches_torch():
    x = np.linspace(-6, 6, 1001)
    np.testing.assert_allclose(elu(x), F.elu(torch.tensor(x)).numpy(), rtol=1e-14, atol=1e-15)


def test_frame_rate_and_shapes():
    """4 * 5 * 6 * 8 * 2 = 1920 samples per latent frame: 24 kHz -> 12.5 Hz."""
    g, _ = read_golden("rates.txt")
    assert 4 * 5 * 6 * 8 * 2 == int(g["sample_rate_hz"]) / float(g["frame_rate_hz"]) == 1920
    w = seanet_weights(seed=0)
    z = encode(audio(1, 2 * 1920)[0], w)
    assert z.shape == (2, 512)
    assert decode(z, w).shape == (2 * 1920,)


def test_encoder_and_decoder_are_causal():
    """Changing samples of frame 2 leaves latent frames 0-1 bit-identical; changing
    latent frame 2 leaves the first 2 * 1920 decoded samples bit-identical."""
    w = seanet_weights(seed=0)
    a = audio(1, 4 * 1920)[0].astype(np.float64)
    z = encode(a, w)
    a2 = a.copy()
    a2[2 * 1920 + 100] += 1.0
    z2 = encode(a2, w)
    np.testing.assert_array_equal(z[:2], z2[:2])
    assert np.abs(z[2:] - z2[2:]).max() > 0
    y = decode(z, w)
    z3 = z.copy()
    z3[2] += 1.0
    y3 = decode(z3, w)
    np.testing.assert_array_equal(y[:2 * 1920], y3[:2 * 1920])
    assert np.abs(y[2 * 1920:] - y3[2 * 1920:]).max() > 0
