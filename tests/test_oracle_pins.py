"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: constants the
pages print (tests/golden/), closed forms, invariants, library routines for the
textbook operations, and brute-force special cases.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from conftest import read_golden
from oracle import (
    ALPHA,
    Oracle,
    Session,
    causal_attention,
    cross_entropy_loss,
    delay_codes,
    joint_sequence,
    rms_norm,
    rope,
    silu,
    top2_margin,
    undelay_codes,
)
from synth import config, generate_weights, param_count, raw_frames

MICRO = config("tiny", name="micro", d_t=64, n_layers_t=2, n_heads_t=4, ffn_t=96, ctx_max=32,
               d_d=32, n_layers_d=2, n_heads_d=2, ffn_d=48, vocab_text=50, codebook=64)


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


# ---------------------------------------------------------------- constants


def test_token_budget_and_frame_rate():
    g, _ = read_golden("rates.txt")
    fr = float(g["frame_rate_hz"])
    bits = math.log2(int(g["codebook_size"]))
    assert bits == 11
    assert fr * int(g["n_codebooks"]) * bits == pytest.approx(float(g["bitrate_bps"]))
    strides = [int(x) for x in g["encoder_strides"].split(",")]
    assert float(g["sample_rate_hz"]) / np.prod(strides) == pytest.approx(fr)
    assert 1000.0 / fr == pytest.approx(float(g["frame_ms"]))
    assert fr * int(g["n_codebooks"]) == float(g["flattened_steps_per_s"])
    assert 5 * 60 * int(g["flattened_steps_per_s"]) == int(g["flattened_steps_5min"])
    cfg = config("b1_7b")
    assert cfg.codebook == int(g["codebook_size"]) and cfg.n_q == int(g["n_codebooks"])


def test_stream_count_and_tokens_per_step():
    g, _ = read_golden("rates.txt")
    cfg = config("tiny")
    fr = raw_frames(cfg, 0, 4)
    V = joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])
    assert V.shape[1] == int(g["n_streams"]) == 2 * cfg.n_q + 1
    # one token per sub-stream and step; without the text stream 2Q remain
    assert V.shape[1] == int(g["tokens_per_step_with_text"])
    assert V.shape[1] - 1 == int(g["tokens_per_step_without_text"])


def test_theoretical_latency_from_delay():
    """A codec frame is complete only after its last acoustic codebook is emitted:
    (1 + delay) frames of 80 ms = 160 ms."""
    g, _ = read_golden("rates.txt")
    tau = int(g["acoustic_delay"])
    T, Q = 6, 8
    frames = np.arange(T * Q).reshape(T, Q) + 1
    model = delay_codes(frames, tau, pad=-1)
    for t in range(T - tau):
        steps = [int(np.argwhere(model[:, q] == frames[t, q])[0, 0]) for q in range(Q)]
        complete_at = max(steps)          # 0-based step that emits the last codebook
        latency = (complete_at - t + 1) * float(g["frame_ms"])
        assert latency == float(g["theoretical_latency_ms"])


def test_param_count_near_pages():
    g, _ = read_golden("rates.txt")
    n = param_count(config("b1_7b"))
    assert abs(n / 1e9 - float(g["total_params_billion"])) / float(g["total_params_billion"]) < 0.02


# ---------------------------------------------------------------- token layout


def test_joint_sequence_matches_fig4_worked_example():
    _, rows = read_golden("fig4_layout_tau1.txt")
    cfg = config("tiny", codebook=2048, delay=1)
    T = 3
    text = np.array([500 + t for t in range(1, T + 1)], dtype=np.int32)
    moshi = np.array([[100 * t + q for q in range(1, 9)] for t in range(1, T + 1)], dtype=np.int32)
    user = np.array([[1000 + 100 * t + q for q in range(1, 9)] for t in range(1, T + 1)], dtype=np.int32)
    V = joint_sequence(cfg, text, moshi, user)
    np.testing.assert_array_equal(V, np.array(rows))


@pytest.mark.parametrize("tau", [0, 1, 2])
def test_delay_roundtrip(tau):
    rng = np.random.default_rng(5)
    x = rng.integers(0, 2048, size=(20, 8)).astype(np.int32)
    m = delay_codes(x, tau, 2048)
    assert (m[:tau, 1:] == 2048).all()
    np.testing.assert_array_equal(m[:, 0], x[:, 0])
    np.testing.assert_array_equal(undelay_codes(m, tau), x[: 20 - tau])


# ---------------------------------------------------------------- primitives


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3.0
    eps = 1e-5
    y = rms_norm(x, np.ones(33), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)
    # scale invariance up to eps, and the gain multiplies elementwise
    g = rng.standard_normal(33)
    np.testing.assert_allclose(rms_norm(x, g, 0.0), rms_norm(5 * x, g, 0.0), rtol=1e-12)
    np.testing.assert_allclose(rms_norm(x, g, eps), y * g, rtol=1e-12)
    # library routine
    t = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), eps)
    np.testing.assert_allclose(rms_norm(x, g, eps), t.numpy(), rtol=1e-12)


def test_rope_closed_form_and_invariants():
    hd, base = 16, 10000.0
    # unit vector on pair i at position m rotates by m * base^(-2i/hd)
    for i in range(hd // 2):
        x = np.zeros((1, 1, hd))
        x[0, 0, 2 * i] = 1.0
        m = 7
        y = rope(x, np.array([m]), base)
        ang = m * base ** (-2.0 * i / hd)
        assert y[0, 0, 2 * i] == pytest.approx(math.cos(ang), abs=1e-14)
        assert y[0, 0, 2 * i + 1] == pytest.approx(math.sin(ang), abs=1e-14)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 3, hd))
    k = rng.standard_normal((1, 3, hd))
    np.testing.assert_allclose(rope(q, np.array([0]), base), q, rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(rope(q, np.array([123]), base)), np.linalg.norm(q), rtol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    def dot(m, n):
        return np.sum(rope(q, np.array([m]), base) * rope(k, np.array([n]), base), axis=-1)
    np.testing.assert_allclose(dot(10, 3), dot(107, 100), rtol=1e-10)
    np.testing.assert_allclose(dot(3, 10), dot(1003, 1010), rtol=1e-10)


def test_rope_matches_complex_rotation():
    """The pair convention equals multiplying (x[2i] + i x[2i+1]) by exp(i m theta_i)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 8))
    pos = np.array([0, 1, 4, 9, 100])
    xc = torch.view_as_complex(torch.from_numpy(x).reshape(5, 3, 4, 2).contiguous())
    theta = 10000.0 ** (-torch.arange(0, 8, 2, dtype=torch.float64) / 8)
    rot = torch.polar(torch.ones(5, 4, dtype=torch.float64), torch.from_numpy(pos)[:, None].double() * theta)
    ref = torch.view_as_real(xc * rot[:, None, :]).reshape(5, 3, 8).numpy()
    np.testing.assert_allclose(rope(x, pos, 10000.0), ref, rtol=1e-12, atol=1e-12)


def test_attention_against_library_and_special_cases():
    rng = np.random.default_rng(3)
    T, H, hd = 6, 2, 8
    q, k, v = (rng.standard_normal((T, H, hd)) for _ in range(3))
    out = causal_attention(q, k, v, np.arange(T))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    # first position sees only itself
    np.testing.assert_allclose(out[0], v[0], rtol=1e-13)
    # equal keys -> uniform weights -> running mean of the values
    kk = np.repeat(k[:1], T, axis=0)
    out2 = causal_attention(q, kk, v, np.arange(T))
    np.testing.assert_allclose(out2, np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None], rtol=1e-12)
    # brute force for one query with a pure-Python softmax
    t, h = 4, 1
    s = [sum(q[t, h, i] * k[p, h, i] for i in range(hd)) / math.sqrt(hd) for p in range(t + 1)]
    w = [math.exp(x - max(s)) for x in s]
    o = [sum(w[p] * v[p, h, i] for p in range(t + 1)) / sum(w) for i in range(hd)]
    np.testing.assert_allclose(out[t, h], o, rtol=1e-12)


def test_silu_library():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0


def test_top2_margin_and_argmax_tie_rule():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [0.5, 0.1, 0.4, 0.2]])
    np.testing.assert_allclose(top2_margin(x), [0.0, 0.1])
    assert int(np.argmax(x[0])) == 1  # lowest index wins a tie


# ---------------------------------------------------------------- model-level invariants


@pytest.fixture(scope="module")
def micro():
    w = generate_weights(MICRO, seed=0, threads=1)
    return Oracle(MICRO, w), w


def _random_V(cfg, S, b=0):
    fr = raw_frames(cfg, b, S)
    return joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])


def test_block_matches_torch_assembly(micro):
    """Temporal + depth pass vs an assembly of torch library layers (F.linear,
    F.rms_norm, complex-number RoPE, scaled_dot_product_attention, F.silu)."""
    m, w = micro
    cfg = MICRO
    S = 9
    V = _random_V(cfg, S)
    lt, la, _ = m.forward_teacher_forced(V)
    F = torch.nn.functional
    T = lambda n: torch.from_numpy(np.asarray(w[n], dtype=np.float64))  # noqa: E731

    def rot(x, pos):  # x [T, H, hd]
        n, H, hd = x.shape
        xc = torch.view_as_complex(x.reshape(n, H, hd // 2, 2).contiguous())
        th = cfg.rope_base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
        r = torch.polar(torch.ones(n, hd // 2, dtype=torch.float64), pos[:, None].double() * th)
        return torch.view_as_real(xc * r[:, None]).reshape(n, H, hd)

    def block(p, h, pos, H):
        n_, d = h.shape
        x = F.rms_norm(h, (d,), T(p + "attn_norm"), cfg.norm_eps)
        q = rot(F.linear(x, T(p + "wq")).reshape(n_, H, -1), pos)
        k = rot(F.linear(x, T(p + "wk")).reshape(n_, H, -1), pos)
        v = F.linear(x, T(p + "wv")).reshape(n_, H, -1)
        a = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                           is_causal=True).transpose(0, 1).reshape(n_, d)
        h = h + F.linear(a, T(p + "wo"))
        x = F.rms_norm(h, (d,), T(p + "ffn_norm"), cfg.norm_eps)
        return h + F.linear(F.silu(F.linear(x, T(p + "w_gate"))) * F.linear(x, T(p + "w_up")), T(p + "w_down"))

    inp = np.concatenate([np.array([[cfg.pad_text] + [cfg.pad_audio] * 16]), V[:-1]])
    h = sum(F.embedding(torch.from_numpy(inp[:, k]).long(), T(f"temporal.emb.{k}")) for k in range(17))
    pos = torch.arange(S)
    for l in range(cfg.n_layers_t):
        h = block(f"temporal.layers.{l}.", h, pos, cfg.n_heads_t)
    z = F.rms_norm(h, (cfg.d_t,), T("temporal.out_norm"), cfg.norm_eps)
    np.testing.assert_allclose(lt, F.linear(z, T("temporal.text_head")).numpy(), rtol=1e-10, atol=1e-12)
    # depth: one frame at a time as a causal sequence of 8 positions, weights by position
    for s in range(S):
        hs = []
        for j in range(cfg.n_q):
            hs.append(F.linear(z[s], T(f"depth.{j}.in_proj")) + T(f"depth.{j}.emb")[int(V[s, j])])
        hd_ = torch.stack(hs)  # [8, d_d]
        for l in range(cfg.n_layers_d):
            # per-position weights: evaluate each position's projections with its own index
            d = cfg.d_d
            H = cfg.n_heads_d
            qs, ks, vs = [], [], []
            for j in range(cfg.n_q):
                p = f"depth.{j}.layers.{l}."
                x = F.rms_norm(hd_[j], (d,), T(p + "attn_norm"), cfg.norm_eps)
                qs.append(F.linear(x, T(p + "wq")))
                ks.append(F.linear(x, T(p + "wk")))
                vs.append(F.linear(x, T(p + "wv")))
            pos8 = torch.arange(cfg.n_q)
            q = rot(torch.stack(qs).reshape(8, H, -1), pos8)
            k = rot(torch.stack(ks).reshape(8, H, -1), pos8)
            v = torch.stack(vs).reshape(8, H, -1)
            a = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                               is_causal=True).transpose(0, 1).reshape(8, d)
            new = []
            for j in range(cfg.n_q):
                p = f"depth.{j}.layers.{l}."
                hj = hd_[j] + F.linear(a[j], T(p + "wo"))
                x = F.rms_norm(hj, (d,), T(p + "ffn_norm"), cfg.norm_eps)
                new.append(hj + F.linear(F.silu(F.linear(x, T(p + "w_gate"))) * F.linear(x, T(p + "w_up")),
                                         T(p + "w_down")))
            hd_ = torch.stack(new)
        for j in range(cfg.n_q):
            ref = F.linear(F.rms_norm(hd_[j], (cfg.d_d,), T(f"depth.{j}.out_norm"), cfg.norm_eps),
                           T(f"depth.{j}.head")).numpy()
            np.testing.assert_allclose(la[s, j], ref, rtol=1e-10, atol=1e-12)


def test_causality(micro):
    m, _ = micro
    S, s0 = 10, 5
    V = _random_V(MICRO, S)
    lt, la, _ = m.forward_teacher_forced(V)
    V2 = V.copy()
    V2[s0:, :] = (V2[s0:, :] + 7) % 40  # perturb frames s0.. (inputs of positions > s0)
    lt2, la2, _ = m.forward_teacher_forced(V2)
    # text logits at frames <= s0 depend on V_0..V_{s0-1} only
    np.testing.assert_array_equal(lt[: s0 + 1], lt2[: s0 + 1])
    np.testing.assert_array_equal(la[:s0], la2[:s0])
    assert not np.allclose(lt[s0 + 1:], lt2[s0 + 1:])


@pytest.mark.parametrize("k", [0, 3, 7])
def test_per_index_depth_isolation(micro, k):
    m, w = micro
    V = _random_V(MICRO, 6)
    lt, la, _ = m.forward_teacher_forced(V)
    w2 = dict(w)
    for name in list(w2):
        if name.startswith(f"depth.{k}."):
            w2[name] = w2[name] * 1.5 if not name.endswith("norm") else w2[name] + 0.5
    m2 = Oracle(MICRO, w2)
    lt2, la2, _ = m2.forward_teacher_forced(V)
    np.testing.assert_array_equal(lt, lt2)
    np.testing.assert_array_equal(la[:, :k], la2[:, :k])
    assert not np.allclose(la[:, k], la2[:, k])


def test_streaming_equals_teacher_forced(micro):
    m, _ = micro
    S = 12
    V = _random_V(MICRO, S)
    lt, la, _ = m.forward_teacher_forced(V)
    sess = Session(m)
    for s in range(S):
        own, l1, l2 = sess.step(V[s, 1 + MICRO.n_q:], force=V[s, : 1 + MICRO.n_q])
        assert _rel(l1, lt[s]) < 1e-12
        assert _rel(l2, la[s]) < 1e-12
        assert own[0] == np.argmax(lt[s])
        for j in range(MICRO.n_q):
            if j >= 1 and s < MICRO.delay:
                assert own[1 + j] == MICRO.pad_audio
            else:
                assert own[1 + j] == np.argmax(la[s, j])


def test_greedy_session_feeds_back_own_tokens(micro):
    m, _ = micro
    S = 6
    fr = raw_frames(MICRO, 0, S)
    user = delay_codes(fr["user"], MICRO.delay, MICRO.pad_audio)
    sess = Session(m)
    toks = []
    for s in range(S):
        own, _, _ = sess.step(user[s])
        toks.append(own)
    V = np.concatenate([np.array(toks), user], axis=1)
    # replaying the generated sequence teacher-forced gives the same argmaxes
    lt, la, _ = m.forward_teacher_forced(V)
    np.testing.assert_array_equal(np.argmax(lt, -1), V[:, 0])
    am = np.argmax(la, -1)
    am[: MICRO.delay, 1:] = MICRO.pad_audio
    np.testing.assert_array_equal(am, V[:, 1:1 + MICRO.n_q])


def test_context_overflow(micro):
    m, _ = micro
    sess = Session(m)
    sess.pos = MICRO.ctx_max
    with pytest.raises(ValueError):
        sess.step(np.zeros(8, dtype=np.int32))


# ---------------------------------------------------------------- loss


def test_cross_entropy_against_library():
    rng = np.random.default_rng(4)
    cfg = MICRO
    B, S = 2, 5
    V = np.stack([_random_V(cfg, S, b) for b in range(B)])
    lt = rng.standard_normal((B, S, cfg.vocab_text))
    la = rng.standard_normal((B, S, cfg.n_q, cfg.codebook))
    out = cross_entropy_loss(cfg, V, lt, la)
    F = torch.nn.functional
    ct = F.cross_entropy(torch.from_numpy(lt.reshape(-1, cfg.vocab_text)), torch.from_numpy(V[..., 0].reshape(-1)).long(),
                         ignore_index=cfg.pad_text).item()
    assert out["ce_text"] == pytest.approx(ct, rel=1e-12)
    per = []
    for j in range(cfg.n_q):
        per.append(F.cross_entropy(torch.from_numpy(la[:, :, j].reshape(-1, cfg.codebook)),
                                   torch.from_numpy(V[..., 1 + j].reshape(-1)).long(),
                                   ignore_index=cfg.pad_audio).item())
    np.testing.assert_allclose(out["ce_per_cb"], per, rtol=1e-12)
    assert out["ce_audio"] == pytest.approx((100 * per[0] + sum(per[1:])) / 107, rel=1e-12)
    assert out["n_audio"] == B * (S * 8 - cfg.delay * 7)


def test_cross_entropy_uniform_logits_closed_form():
    cfg = MICRO
    V = _random_V(cfg, 4)[None]
    out = cross_entropy_loss(cfg, V, np.zeros((1, 4, cfg.vocab_text)), np.zeros((1, 4, 8, cfg.codebook)))
    assert out["ce_text"] == pytest.approx(math.log(cfg.vocab_text), rel=1e-14)
    assert out["ce_audio"] == pytest.approx(math.log(cfg.codebook), rel=1e-14)
    assert out["ce_total"] == pytest.approx(math.log(cfg.vocab_text) + math.log(cfg.codebook), rel=1e-14)
    assert ALPHA[0] == 100 and (ALPHA[1:] == 1).all()


def test_text_logit_scale():
    """With unit-RMS z and N(0, 0.02^2) head weights the text logits have std
    0.02 * sqrt(d) (here 0.02 * 16 = 0.32)."""
    cfg = config("tiny", vocab_text=32000, n_layers_t=1)
    w = generate_weights(cfg, threads=4)
    m = Oracle(cfg, w)
    V = _random_V(cfg, 2)
    lt, _, z = m.forward_teacher_forced(V, depth=False)
    np.testing.assert_allclose(np.mean(z * z, axis=-1), 1.0, rtol=1e-3)
    assert np.std(lt) == pytest.approx(0.02 * math.sqrt(cfg.d_t), rel=0.02)
