"""Oracle pins for Mimi's bottleneck Transformer. All on the CPU."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.mimi_transformer import forward, gelu, layer_norm, rope, window_attention
from synth.mimi_inputs import mimi_weights

D, H, FF = 64, 4, 128  # small shapes for the CPU


def _w(n_layers=2, scale=0.5, seed=0):
    return mimi_weights(n_layers, D, FF, seed=seed, scale=scale)


def test_layer_norm_and_gelu_match_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((9, 33)) * 3 + 1
    g, b = rng.standard_normal(33), rng.standard_normal(33)
    ref = F.layer_norm(torch.tensor(x), (33,), torch.tensor(g), torch.tensor(b), eps=1e-5).numpy()
    np.testing.assert_allclose(layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-12)
    y = rng.standard_normal(1000) * 4
    np.testing.assert_allclose(gelu(y), F.gelu(torch.tensor(y), approximate="none").numpy(), rtol=1e-12, atol=1e-14)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3, 16))
    z = torch.view_as_complex(torch.tensor(x).reshape(7, 3, 8, 2).contiguous())
    ang = torch.arange(7, dtype=torch.float64)[:, None] * 10000.0 ** (-2.0 * torch.arange(8, dtype=torch.float64) / 16)[None, :]
    ref = torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)[:, None, :]).reshape(7, 3, 16).numpy()
    np.testing.assert_allclose(rope(x), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [1, 5, 250])
def test_window_attention_matches_masked_sdpa(window):
    rng = np.random.default_rng(2)
    S, Hh, hd = 20, 2, 8
    q, k, v = (rng.standard_normal((S, Hh, hd)) for _ in range(3))
    t = torch.arange(S)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - window)
    ref = F.scaled_dot_product_attention(*(torch.tensor(a).transpose(0, 1) for a in (q, k, v)), attn_mask=mask)
    np.testing.assert_allclose(window_attention(q, k, v, window), ref.transpose(0, 1).numpy(), rtol=1e-10,
                               atol=1e-12)


def test_block_matches_torch_assembly():
    """One layer against torch library layers (layer_norm, linear, complex RoPE,
    masked SDPA, gelu)."""
    w = _w(1)
    S, window = 12, 5
    x = np.random.default_rng(3).standard_normal((S, D))
    T = {k.rsplit(".", 1)[1]: torch.tensor(v, dtype=torch.float64) for k, v in w.items()}
    h = torch.tensor(x)
    n = F.layer_norm(h, (D,), T["ln1_g"], T["ln1_b"], eps=1e-5)

    def rot(a):
        z = torch.view_as_complex(a.reshape(S, H, D // H // 2, 2).contiguous())
        i = torch.arange(D // H // 2, dtype=torch.float64)
        ang = torch.arange(S, dtype=torch.float64)[:, None] * 10000.0 ** (-2.0 * i / (D // H))[None, :]
        return torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)[:, None, :]).reshape(S, H, D // H)

    q, k = rot(F.linear(n, T["wq"])), rot(F.linear(n, T["wk"]))
    v = F.linear(n, T["wv"]).reshape(S, H, D // H)
    t = torch.arange(S)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - window)
    a = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), attn_mask=mask)
    h = h + T["scale1"] * F.linear(a.transpose(0, 1).reshape(S, D), T["wo"])
    n = F.layer_norm(h, (D,), T["ln2_g"], T["ln2_b"], eps=1e-5)
    h = h + T["scale2"] * F.linear(F.gelu(F.linear(n, T["w1"])), T["w2"])
    np.testing.assert_allclose(forward(x, w, 1, H, window), h.numpy(), rtol=1e-10, atol=1e-10)


def test_causal_and_windowed_receptive_field():
    """Perturbing frame p changes no output before p; with one layer and window 5,
    none from p + 5 on."""
    w = _w(1)
    S, window, p = 16, 5, 4
    x = np.random.default_rng(4).standard_normal((S, D))
    y = forward(x, w, 1, H, window)
    x2 = x.copy()
    x2[p] += 1.0
    y2 = forward(x2, w, 1, H, window)
    np.testing.assert_array_equal(y[:p], y2[:p])
    np.testing.assert_array_equal(y[p + window:], y2[p + window:])
    assert np.abs(y[p:p + window] - y2[p:p + window]).max() > 1e-3


def test_zero_layerscale_is_identity():
    w = _w(2)
    for k in w:
        if "scale" in k:
            w[k] = np.zeros_like(w[k])
    x = np.random.default_rng(5).standard_normal((6, D))
    np.testing.assert_array_equal(forward(x, w, 2, H, 250), x)
