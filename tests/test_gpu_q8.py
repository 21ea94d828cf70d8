"""GPU parity of the 8-bit block weight format (block-32 asymmetric MinMax, fp16
scale and min): the library's quantiser against the oracle's, code for code; the
mid configuration streamed after a 375-frame prompt against the oracle run on the
quantise-dequantise image of the weights; the 7B shape at batch 1 on sampled
frames."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import Oracle, Session, dequantize_q8, is_linear, quantize_q8
from parity_util import compare_frame, prompt_V
from synth import config, generate_weights

pytestmark = pytest.mark.gpu

TOL = 1e-2  # bf16 activations' bar; the dequantised weights are exact in both


def dequantized(w):
    """The oracle's quantise-dequantise image of every linear map, tensors in parallel."""
    names = [n for n in w if is_linear(n)]
    with ThreadPoolExecutor(16) as ex:
        done = dict(zip(names, ex.map(lambda n: dequantize_q8(*quantize_q8(w[n])), names)))
    return {n: done.get(n, w[n]) for n in w}


def oracle_prefilled(model, V, P):
    sess = Session(model)
    model.temporal(np.concatenate([model.initial_frame[None], V[:P - 1]]), 0, sess.cache)
    sess.pos = P
    sess.prev = V[P - 1].copy()
    return sess


def test_q8_codes_match_oracle_quantiser():
    from full_duplex_speech_amd import Moshi, moshi_read_q8
    cfg = config("mid_q8")
    w = generate_weights(cfg, seed=0)
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    names = [n for n in w if is_linear(n)]
    assert len(names) >= 8 * 6 + 1
    for name in names:
        q, s, m = quantize_q8(w[name])
        gq, gs, gm = moshi_read_q8(eng.ctx, name, *w[name].shape)
        assert np.array_equal(gq, q), name
        assert np.array_equal(gs.view(np.uint16), s.view(np.uint16)), name
        assert np.array_equal(gm.view(np.uint16), m.view(np.uint16)), name
    eng.close()
    print(f"mid_q8: {len(names)} linear maps, codes and block parameters identical")


def test_q8_mid_prompt_then_generate():
    from full_duplex_speech_amd import Moshi
    cfg = config("mid_q8")
    P, n = cfg.prompt_frames, cfg.gen_frames
    w = generate_weights(cfg, seed=0)
    model = Oracle(cfg, dequantized(w))
    V = prompt_V(cfg, 0, P + n)
    sess = oracle_prefilled(model, V, P)
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    eng.forward_teacher_forced(V[None, :P], fill_kv=True, skip_depth=True, logits=False, loss=False)
    worst, checked, total = 0.0, 0, 0
    for s in range(n):
        own, lt, la = sess.step(V[P + s, 9:])
        tok, glt, gla = eng.step(V[P + s, 9:][None], force=own[None], logits=True)
        wv, c, t = compare_frame(cfg, P + s, own, lt, la, tok[0], glt[0], gla[0], TOL)
        worst, checked, total = max(worst, wv), checked + c, total + t
    eng.close()
    print(f"mid_q8 P={P}: {n} frames, worst rel-L2 {worst:.2e}, tokens checked {checked}/{total}")


def test_q8_mid_free_running_matches_greedy():
    """Without forcing, the library's own greedy tokens drive the stream; they agree
    with the oracle's wherever the oracle's top-2 margin is clear."""
    from full_duplex_speech_amd import Moshi
    cfg = config("mid_q8")
    P, n = 24, 16
    w = generate_weights(cfg, seed=1)
    model = Oracle(cfg, dequantized(w))
    V = prompt_V(cfg, 0, P + n, seed=1)
    sess = oracle_prefilled(model, V, P)
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    eng.forward_teacher_forced(V[None, :P], fill_kv=True, skip_depth=True, logits=False, loss=False)
    for s in range(n):
        own, lt, la = sess.step(V[P + s, 9:])
        tok, glt, gla = eng.step(V[P + s, 9:][None], logits=True)
        compare_frame(cfg, P + s, own, lt, la, tok[0], glt[0], gla[0], TOL)
        if not np.array_equal(tok[0], own):
            break  # a tie broken the other way: the streams part from here
    eng.close()


def test_q8_7b_batch1_after_full_prompt():
    from full_duplex_speech_amd import Moshi
    cfg = config("b1_7b_q8")
    P, n = cfg.prompt_frames, 3
    w = generate_weights(cfg, seed=0)
    model = Oracle(cfg, dequantized(w), dtype=np.float32)
    V = prompt_V(cfg, 0, P + n)
    sess = oracle_prefilled(model, V, P)
    ref = [sess.step(V[P + s, 9:]) for s in range(n)]
    del model, sess
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    eng.forward_teacher_forced(V[None, :P], fill_kv=True, skip_depth=True, logits=False, loss=False)
    worst = 0.0
    for s in range(n):
        own, lt, la = ref[s]
        tok, glt, gla = eng.step(V[P + s, 9:][None], force=own[None], logits=True)
        wv, _, _ = compare_frame(cfg, P + s, own, lt, la, tok[0], glt[0], gla[0], TOL)
        worst = max(worst, wv)
    eng.close()
    print(f"7B q8 b1: worst rel-L2 {worst:.2e}")
