"""The seeded input generator: determinism, shapes, bf16 rounding."""
import numpy as np
import torch

from synth import bf16_round, config, generate_weight, generate_weights, raw_frames, weight_specs


def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([(rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], np.float32)])
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_round(x.copy()), ref)


def test_weights_deterministic_and_threaded_equal():
    cfg = config("tiny")
    a = generate_weights(cfg, seed=0, threads=1)
    b = generate_weights(cfg, seed=0, threads=4)
    assert list(a) == [n for n, _, _ in weight_specs(cfg)]
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
        assert a[n].dtype == np.float32
    np.testing.assert_array_equal(generate_weight(cfg, 20), a[weight_specs(cfg)[20][0]])
    c = generate_weights(cfg, seed=1, threads=2)
    assert not np.array_equal(a["temporal.layers.0.wq"], c["temporal.layers.0.wq"])


def test_weight_statistics_and_bf16_values():
    cfg = config("tiny", dtype="bf16")
    w = generate_weights(cfg, threads=2)
    wq = w["temporal.layers.1.wq"]
    assert abs(wq.std() - 0.02) < 0.001
    assert abs(w["temporal.emb.3"].std() - 1.0) < 0.02
    assert (w["temporal.layers.0.attn_norm"] == 1).all()
    assert (wq.view(np.uint32) & 0xFFFF == 0).all()


def test_raw_frames_ranges():
    cfg = config("tiny")
    fr = raw_frames(cfg, 3, 100)
    assert fr["text"].min() >= 0 and fr["text"].max() < cfg.vocab_text
    for k in ("moshi", "user"):
        assert fr[k].shape == (100, cfg.n_q)
        assert fr[k].min() >= 0 and fr[k].max() < cfg.codebook
    np.testing.assert_array_equal(raw_frames(cfg, 3, 100)["user"], fr["user"])
    assert not np.array_equal(raw_frames(cfg, 4, 100)["user"], fr["user"])
