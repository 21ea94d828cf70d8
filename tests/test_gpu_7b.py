"""GPU parity at the 7B shape (bf16 weights), on sampled outputs the float32
oracle can compute: batch 1 after the full 375-frame prompt; batch 8 with short
prompts (all eight conversations, independently seeded); teacher-forced logits
and loss at the first frames of four sequences."""
import numpy as np
import pytest

from oracle import Oracle, Session
from parity_util import compare_frame, prompt_V, rel_l2
from synth import config, generate_weights

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def setup():
    cfg = config("b1_7b")
    w = generate_weights(cfg, seed=0)
    return cfg, w, Oracle(cfg, w, dtype=np.float32)


def oracle_prefilled(model, V, P):
    sess = Session(model)
    if P:
        model.temporal(np.concatenate([model.initial_frame[None], V[:P - 1]]), 0, sess.cache)
        sess.pos = P
        sess.prev = V[P - 1].copy()
    return sess


def test_7b_batch1_after_full_prompt(setup):
    from full_duplex_speech_amd import Moshi
    cfg, w, model = setup
    P, n = cfg.prompt_frames, 4
    V = prompt_V(cfg, 0, P + n)
    sess = oracle_prefilled(model, V, P)
    ref = [sess.step(V[P + s, 9:]) for s in range(n)]
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
    print(f"7B b1: worst rel-L2 {worst:.2e}")


def test_7b_batch8_short_prompts(setup):
    from full_duplex_speech_amd import Moshi
    cfg, w, model = setup
    B, P, n = 8, 24, 2
    Vs = [prompt_V(cfg, b, P + n) for b in range(B)]
    refs = []
    for b in range(B):
        sess = oracle_prefilled(model, Vs[b], P)
        refs.append([sess.step(Vs[b][P + s, 9:]) for s in range(n)])
    eng = Moshi(cfg, max_batch=B)
    eng.load_weights(w)
    eng.forward_teacher_forced(np.stack([v[:P] for v in Vs]), fill_kv=True, skip_depth=True, logits=False,
                               loss=False)
    worst = 0.0
    for s in range(n):
        user = np.stack([Vs[b][P + s, 9:] for b in range(B)])
        force = np.stack([refs[b][s][0] for b in range(B)])
        tok, glt, gla = eng.step(user, force=force, logits=True)
        for b in range(B):
            own, lt, la = refs[b][s]
            wv, _, _ = compare_frame(cfg, P + s, own, lt, la, tok[b], glt[b], gla[b], TOL)
            worst = max(worst, wv)
    eng.close()
    print(f"7B b8: worst rel-L2 {worst:.2e}")


def test_7b_teacher_forced_first_frames(setup):
    from full_duplex_speech_amd import Moshi
    from oracle import cross_entropy_loss
    cfg, w, model = setup
    B, S = 4, 6
    V = np.stack([prompt_V(cfg, b, S) for b in range(B)])
    eng = Moshi(cfg, max_batch=B)
    eng.load_weights(w)
    lt, la, loss = eng.forward_teacher_forced(V)
    eng.close()
    rt, ra = zip(*[model.forward_teacher_forced(V[b])[:2] for b in range(B)])
    rt, ra = np.stack(rt), np.stack(ra)
    wt = max(rel_l2(lt[b, s], rt[b, s]) for b in range(B) for s in range(S))
    wa = np.array([[[rel_l2(la[b, s, j], ra[b, s, j]) for j in range(8)] for s in range(S)] for b in range(B)])
    print(f"7B teacher-forced: text worst {wt:.2e}; audio worst {wa.max():.2e} per codebook {wa.max(axis=(0, 1))}; "
          f"whole-tensor text {rel_l2(lt, rt):.2e} audio {rel_l2(la, ra):.2e}")
    worst = max(wt, wa.max())
    assert worst <= TOL
    ref = cross_entropy_loss(cfg, V, rt, ra)
    for k in ("ce_text", "ce_audio", "ce_total"):
        assert loss[k] == pytest.approx(ref[k], rel=1e-3)
    print(f"7B teacher-forced: worst rel-L2 {worst:.2e}, ce_total {loss['ce_total']:.4f}")
