"""GPU parity of the 16-index depth (the user's codebooks predicted after Moshi's):
simulated dialogues with no user input, greedy and sampled, with the oracle
shadowing the library on the library's own tokens; given user codes; and the
teacher-forced pass of a 16-index model over Moshi's codebooks."""
import numpy as np
import pytest

from oracle import Oracle, Session, joint_sequence, top2_margin
from parity_util import MARGIN, rel_l2
from synth import config, generate_weights, raw_frames
from test_gpu_sampling import check_draw

pytestmark = pytest.mark.gpu

TOLS = {"f32": 1e-4, "bf16": 1e-2}


@pytest.mark.parametrize("name,n,temps", [("tiny_sim", 40, (0.0, 0.0)), ("mid_sim", 16, (0.0, 0.0)),
                                          ("tiny_sim", 30, (0.7, 0.8))])
def test_simulated_dialogue(name, n, temps):
    from full_duplex_speech_amd import Moshi
    cfg = config(name)
    tol = TOLS[cfg.dtype]
    w = generate_weights(cfg, seed=0)
    model = Oracle(cfg, w)
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    seed = 4321
    eng.set_sampling(*temps, seed)
    sess = Session(model)
    checked = exact = 0
    for s in range(n):
        tok, glt, gla = eng.step(1, logits=True)        # no user input
        assert tok.shape == (1, 17) and gla.shape == (1, 16, cfg.codebook)
        own, lt, la = sess.step(tok[0, 9:], force=tok[0, :9])
        worst = max(rel_l2(glt[0], lt), max(rel_l2(gla[0, j], la[j]) for j in range(16)))
        assert worst <= tol, (s, worst)
        for j in range(16):
            if j % 8 and s < cfg.delay:
                assert tok[0, 1 + j] == cfg.pad_audio
            elif temps[1] > 0:
                exact += check_draw(tok[0, 1 + j], gla[0, j], temps[1], seed, s, 0, j + 1)
            elif top2_margin(la[j]) > MARGIN:
                checked += 1
                assert tok[0, 1 + j] == own[1 + j], (s, j)
    eng.close()
    print(f"{name} temps {temps}: {n} simulated frames, audio tokens checked {checked}, exact draws {exact}")


def test_given_user_codes_and_teacher_forced():
    from full_duplex_speech_amd import Moshi
    from oracle import cross_entropy_loss
    cfg = config("tiny_sim")
    w = generate_weights(cfg, seed=0)
    model = Oracle(cfg, w)
    fr = raw_frames(cfg, 0, 12, seed=9)
    V = joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    sess = Session(model)
    for s in range(12):
        tok, glt, gla = eng.step(V[s, 9:][None], force=V[s, :9][None], logits=True)
        own, lt, la = sess.step(V[s, 9:], force=V[s, :9])
        assert rel_l2(glt[0], lt) <= 1e-4 and max(rel_l2(gla[0, j], la[j]) for j in range(16)) <= 1e-4
        for j in range(16):
            if not (j % 8 and s < cfg.delay) and top2_margin(la[j]) > MARGIN:
                assert tok[0, 1 + j] == own[1 + j]
    # teacher-forced scoring of a 16-index model covers Moshi's codebooks
    eng.reset()
    lt, la, loss = eng.forward_teacher_forced(V[None])
    rt, ra, _ = model.forward_teacher_forced(V)
    assert la.shape[2] == 8
    assert rel_l2(lt[0], rt) <= 1e-4 and rel_l2(la[0], ra[:, :8]) <= 1e-4
    ref = cross_entropy_loss(cfg, V[None], rt[None], ra[None, :, :8])
    assert loss["ce_total"] == pytest.approx(ref["ce_total"], rel=1e-5)
    eng.close()
