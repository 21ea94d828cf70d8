"""GPU parity of temperature sampling (Philox4x64-10 + Gumbel-max, float32).

The library samples its own tokens; the oracle shadows each conversation, forced
with the library's tokens so both stay on one sequence. Logits are compared as
usual. Every drawn token is checked against the oracle's draw from the library's
own float32 logits: it must be the oracle's pick wherever the two best perturbed
scores differ by more than 1e-4, and within 1e-4 of the best score otherwise
(the device and NumPy logarithms may differ in the last bit)."""
import numpy as np
import pytest

from oracle import Oracle, Session, TtsTextControl, joint_sequence
from oracle.sampling import sample, scores, uniforms
from parity_util import rel_l2
from synth import config, generate_weights, raw_frames

pytestmark = pytest.mark.gpu

EPS = 1e-4


def check_draw(tok, logits, T, seed, pos, conv, slot):
    l32 = np.asarray(logits, dtype=np.float32)
    s = scores(l32, T, uniforms(len(l32), seed, pos, conv, slot))
    best = float(s.max())
    assert float(s[tok]) >= best - EPS * max(1.0, abs(best)), (pos, conv, slot, tok)
    top = np.sort(s)[-2:]
    if top[1] - top[0] > EPS * max(1.0, abs(best)):
        assert tok == int(np.argmax(s)), (pos, conv, slot, tok, int(np.argmax(s)))
        return 1
    return 0


@pytest.mark.parametrize("name,B,n,tol", [("tiny", 2, 30, 1e-4), ("mid_bf16", 1, 12, 1e-2)])
def test_sampled_stream(name, B, n, tol):
    from full_duplex_speech_amd import Moshi
    cfg = config(name)
    tt, ta, seed = 0.7, 0.8, 1234
    w = generate_weights(cfg, seed=0)
    model = Oracle(cfg, w)
    Vs = []
    for b in range(B):
        fr = raw_frames(cfg, b, n, seed=5)
        Vs.append(joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"]))
    sessions = [Session(model, conversation=b) for b in range(B)]
    eng = Moshi(cfg, max_batch=B)
    eng.load_weights(w)
    eng.set_sampling(tt, ta, seed)
    exact = differs = 0
    for s in range(n):
        user = np.stack([Vs[b][s, 9:] for b in range(B)])
        tok, glt, gla = eng.step(user, logits=True)
        for b in range(B):
            _, lt, la = sessions[b].step(user[b], force=tok[b])
            assert rel_l2(glt[b], lt) <= tol and max(rel_l2(gla[b, j], la[j]) for j in range(8)) <= tol
            exact += check_draw(tok[b, 0], glt[b], tt, seed, s, b, 0)
            differs += int(tok[b, 0] != np.argmax(glt[b]))
            for j in range(8):
                if j >= 1 and s < cfg.delay:
                    assert tok[b, 1 + j] == cfg.pad_audio
                    continue
                exact += check_draw(tok[b, 1 + j], gla[b, j], ta, seed, s, b, j + 1)
    eng.close()
    assert differs > 0  # the draws are not the greedy tokens
    print(f"{name}: {n} sampled frames x {B}, {exact} draws matched exactly, {differs} text draws off argmax")


def test_sampling_off_is_greedy_and_reseeding_repeats():
    """Temperature 0 restores greedy decoding; the same seed replays the same draws."""
    from full_duplex_speech_amd import Moshi
    cfg = config("tiny")
    w = generate_weights(cfg, seed=0)
    fr = raw_frames(cfg, 0, 10, seed=2)
    V = joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    runs = []
    for temps in [(0.8, 0.8), (0.8, 0.8), (0.0, 0.0)]:
        eng.reset()
        eng.set_sampling(*temps, seed=99)
        out = []
        for s in range(10):
            tok, glt, gla = eng.step(V[s, 9:][None], logits=True)
            if temps[0] == 0:
                assert tok[0, 0] == np.argmax(glt[0])
                assert all(tok[0, 1 + j] == np.argmax(gla[0, j]) for j in range(8) if not (j and s < cfg.delay))
            out.append(tok[0].copy())
        runs.append(np.array(out))
    np.testing.assert_array_equal(runs[0], runs[1])
    assert not np.array_equal(runs[0], runs[2])
    from full_duplex_speech_amd import MoshiError
    with pytest.raises(MoshiError):
        eng.set_sampling(-0.5, 0.8, 1)
    eng.close()


def test_sampled_tts_text_control():
    """TTS at temperature 0.6 (the pages' TTS setting): the library's text choices equal
    the oracle's control replayed with the oracle's sampler on the library's logits."""
    from full_duplex_speech_amd import Moshi
    cfg = config("tiny_tts")
    n, T, seed = 50, 0.6, 77
    w = generate_weights(cfg, seed=0)
    model = Oracle(cfg, w)
    words = [[5, 6], [7], [8, 9, 10], [11], [12, 13]]
    pad, epad, bonus = 0, 1, 6.0
    eng = Moshi(cfg, max_batch=1, tts_max_tokens=16)
    eng.load_weights(w)
    eng.set_sampling(T, 0.8, seed)
    eng.tts_text(words, pad, epad, 0.65, bonus)
    sess = Session(model)
    user = np.full(8, cfg.pad_audio, dtype=np.int32)
    text_seq, text_logits = [], []
    for s in range(n):
        tok, glt, gla = eng.step(user[None], logits=True)
        _, lt, la = sess.step(user, force=tok[0])
        assert rel_l2(glt[0], lt) <= 1e-4
        text_seq.append(int(tok[0, 0]))
        text_logits.append(glt[0].copy())
    eng.close()
    replay = TtsTextControl(words, pad, epad, 0.65, bonus)
    got = [replay.choose(l, lambda lg, s=s: sample(lg, T, seed, s, 0, 0)) for s, l in enumerate(text_logits)]
    assert got == text_seq
    fed = [t for t in text_seq if t not in (pad, epad)]
    assert fed == [t for wd in words for t in wd][:len(fed)] and fed and pad in text_seq
