"""Oracle pins for the streaming modes: text-audio delay (ASR and TTS layouts),
per-slot forcing, the text-only (depth-free) ASR step and the zero-shot TTS text
control. All on the CPU."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import Oracle, Session, TtsTextControl, joint_sequence, stream_starts
from synth import config, generate_weights, raw_frames

MICRO = config("tiny", name="micro", d_t=64, n_layers_t=2, n_heads_t=4, ffn_t=96, ctx_max=32,
               d_d=32, n_layers_d=2, n_heads_d=2, ffn_d=48, vocab_text=50, codebook=64)


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


@pytest.fixture(scope="module")
def weights():
    return generate_weights(MICRO, seed=0, threads=1)


def _symbolic(T):
    text = np.array([500 + t for t in range(1, T + 1)], dtype=np.int32)
    moshi = np.array([[100 * t + q for q in range(1, 9)] for t in range(1, T + 1)], dtype=np.int32)
    user = np.array([[1000 + 100 * t + q for q in range(1, 9)] for t in range(1, T + 1)], dtype=np.int32)
    return text, moshi, user


@pytest.mark.parametrize("fixture", ["fig8_asr_layout.txt", "fig9_tts_layout.txt"])
def test_joint_sequence_matches_asr_tts_worked_examples(fixture):
    g, rows = read_golden(fixture)
    cfg = config("tiny", codebook=2048, delay=int(g["acoustic_delay"]), text_delay=int(g["text_delay"]))
    V = joint_sequence(cfg, *_symbolic(len(rows)))
    np.testing.assert_array_equal(V, np.array(rows))


def test_two_second_delay_is_25_frames():
    """The ASR/TTS configurations put text and audio 2 s apart at the codec's frame rate."""
    g, _ = read_golden("rates.txt")
    frames = 2.0 * float(g["frame_rate_hz"])
    assert config("b1_7b_asr").text_delay == frames == -config("b1_7b_tts").text_delay
    assert config("b1_7b_asr").delay == config("b1_7b_tts").delay == 2


def test_zero_text_delay_is_the_dialogue_layout():
    cfg = config("tiny")
    fr = raw_frames(cfg, 0, 9)
    base = joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])
    assert stream_starts(cfg) == (0, 0)
    for d in (4, -4):
        V = joint_sequence(cfg.replace(text_delay=d), fr["text"], fr["moshi"], fr["user"])
        if d > 0:  # only the text moves
            np.testing.assert_array_equal(V[:, 1:], base[:, 1:])
            np.testing.assert_array_equal(V[d:, 0], base[:-d, 0])
            assert (V[:d, 0] == cfg.pad_text).all()
        else:  # only the audio moves
            np.testing.assert_array_equal(V[:, 0], base[:, 0])
            np.testing.assert_array_equal(V[-d:, 1:], base[:d, 1:])
            assert (V[:-d, 1:] == cfg.pad_audio).all()


def test_unforced_slots_equal_no_forcing(weights):
    m = Oracle(MICRO, weights)
    V = joint_sequence(MICRO, *[raw_frames(MICRO, 0, 6)[k] for k in ("text", "moshi", "user")])
    a, b = Session(m), Session(m)
    for s in range(6):
        o1, t1, a1 = a.step(V[s, 9:])
        o2, t2, a2 = b.step(V[s, 9:], force=np.full(9, -1))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(t1, t2)
        np.testing.assert_array_equal(a1, a2)


def test_asr_text_only_stream_equals_teacher_forced(weights):
    """ASR: audio forced, text greedy, depth skipped. The text logits are bit-identical
    to those of full steps with the same forcing, and match a teacher-forced pass over
    the realised sequence; the text is pad until the text stream starts."""
    cfg = MICRO.replace(delay=2, text_delay=3)
    m = Oracle(cfg, weights)
    S = 12
    fr = raw_frames(cfg, 0, S)
    V = joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])
    fast, full = Session(m), Session(m)
    lts, realised = [], []
    for s in range(S):
        force = np.full(9, -1)
        force[1:] = V[s, 1:9]
        own, lt, la = fast.step(V[s, 9:], force=force, text_only=True)
        own_f, lt_f, _ = full.step(V[s, 9:], force=force)
        assert la is None
        np.testing.assert_array_equal(lt, lt_f)
        assert own[0] == own_f[0]
        np.testing.assert_array_equal(own[1:], V[s, 1:9])
        assert own[0] == (cfg.pad_text if s < 3 else np.argmax(lt))
        lts.append(lt)
        realised.append(np.concatenate([own[:1], V[s, 1:]]))
    lt_tf, _, _ = m.forward_teacher_forced(np.array(realised), depth=False)
    assert max(_rel(lts[s], lt_tf[s]) for s in range(S)) < 1e-12


def test_text_only_without_forced_audio_stores_pad(weights):
    m = Oracle(MICRO, weights)
    sess = Session(m)
    force = np.full(9, -1)
    force[2] = 7
    own, _, _ = sess.step(np.full(8, MICRO.pad_audio), force=force, text_only=True)
    assert own[2] == 7 and (np.delete(own[1:], 1) == MICRO.pad_audio).all()
    assert sess.prev[2] == 7 and sess.prev[1] == MICRO.pad_audio


def test_tts_stream_equals_teacher_forced(weights):
    """TTS: the text control picks the text, the audio is greedy. The audio logits
    match a teacher-forced pass over the realised sequence, the audio tokens are its
    argmax once each codebook's stream has started and pad before; the text tokens
    are the control's decisions, replayed on the same logits."""
    cfg = MICRO.replace(delay=2, text_delay=-3)
    m = Oracle(cfg, weights)
    S = 12
    words = [[3, 4], [5], [6, 7, 8], [9]]
    ctl = TtsTextControl(words, pad_id=0, epad_id=1, target_pad_ratio=0.5, bonus=0.5)
    sess = Session(m)
    user = np.full((S, 8), cfg.pad_audio, dtype=np.int32)
    outs, realised = [], []
    for s in range(S):
        own, lt, la = sess.step(user[s], text_choice=ctl.choose)
        outs.append((own, lt, la))
        realised.append(np.concatenate([own, user[s]]))
    R = np.array(realised)
    _, la_tf, _ = m.forward_teacher_forced(R)
    starts = [3] + [5] * 7
    for s, (own, lt, la) in enumerate(outs):
        assert _rel(la, la_tf[s]) < 1e-12
        for j in range(8):
            assert own[1 + j] == (cfg.pad_audio if s < starts[j] else np.argmax(la_tf[s, j]))
    replay = TtsTextControl(words, pad_id=0, epad_id=1, target_pad_ratio=0.5, bonus=0.5)
    assert [replay.choose(lt) for _, lt, _ in outs] == [int(o[0]) for o, _, _ in outs]
    fed = [t for t in R[:, 0] if t not in (0, 1)]
    assert fed == [t for w in words for t in w][:len(fed)]


def test_tts_text_control_decisions():
    """Each rule of the TTS text control on hand-made logits (vocabulary of 10,
    PAD = 0, EPAD = 1, target padding ratio 0.5, bonus 2)."""
    ctl = TtsTextControl([[5, 6], [7], [8, 9]], pad_id=0, epad_id=1, target_pad_ratio=0.5, bonus=2.0)

    def lg(**kv):
        v = np.zeros(10, dtype=np.float32)
        for k, x in kv.items():
            v[int(k[1:])] = x
        return v

    steps = [
        (lg(i3=3.0), 5),            # 0 pads of 0: bonus (PAD 2.0) loses to 3.0 -> first word starts
        (lg(i3=9.0), 6),            # inside the word: its next token, logits not consulted
        (lg(i4=1.5), 0),            # 0 < 0.5*2: PAD with bonus 2.0 beats 1.5
        (lg(i1=2.5), 1),            # EPAD 2.5 beats PAD 2.0 and is taken
        (lg(i3=2.0), 0),            # PAD 2.0 ties token 3 at 2.0: the lower index wins
        (lg(i2=5.0), 7),            # 2 < 0.5*5: bonus, but token 2 wins -> next word
        (lg(i0=-5.0, i9=0.1), 8),   # PAD -3.0 with bonus; token 9 wins -> next word
        (lg(), 9),                  # inside the word
        (lg(i5=3.0), 0),            # every word fed: PAD
        (lg(i6=1.0), 0),            # 3 < 0.5*9: PAD 2.0 beats 1.0
    ]
    got = [ctl.choose(l) for l, _ in steps]
    assert got == [want for _, want in steps]
    assert ctl.n_pad == 4 and ctl.n_steps == 10


def test_tts_text_control_bonus_only_below_target():
    ctl = TtsTextControl([[5], [6]], pad_id=0, epad_id=1, target_pad_ratio=0.25, bonus=1.0)
    z = np.zeros(10, dtype=np.float32)
    z[3] = 0.5
    assert ctl.choose(z) == 0        # first step: 0 < 0.25 -> PAD 1.0 beats 0.5
    assert ctl.choose(z) == 5        # 1 pad of 1: at target, no bonus -> next word
    assert ctl.choose(z) == 6        # 1 of 2 >= 0.5: no bonus
    assert ctl.choose(z) == 0        # 1 of 3 >= 0.75: no bonus, but nothing left: PAD
    with pytest.raises(ValueError):
        TtsTextControl([[5]], pad_id=0, epad_id=1, target_pad_ratio=0.5, bonus=-1.0)
    with pytest.raises(ValueError):
        TtsTextControl([[5], []], pad_id=0, epad_id=1, target_pad_ratio=0.5, bonus=1.0)


# ---------------------------------------------------------------- 16-index depth

SIM = MICRO.replace(name="micro_sim", n_depth=16)


def test_sixteen_index_depth_leaves_moshi_unchanged():
    """The user's indices come after Moshi's in the depth chain: with the user's codes
    given, text and Moshi's audio logits and tokens are bit-identical to the 8-index model
    with the same weights."""
    w16 = generate_weights(SIM, seed=0, threads=1)
    w8 = {k: v for k, v in w16.items() if not k.startswith("depth.") or int(k.split(".")[1]) < 8}
    m8, m16 = Oracle(MICRO, w8), Oracle(SIM, w16)
    fr = raw_frames(MICRO, 0, 8)
    V = joint_sequence(MICRO, fr["text"], fr["moshi"], fr["user"])
    a, b = Session(m8), Session(m16)
    for s in range(8):
        o8, t8, a8 = a.step(V[s, 9:])
        o16, t16, a16 = b.step(V[s, 9:])
        assert o16.shape == (17,) and a16.shape == (16, MICRO.codebook)
        np.testing.assert_array_equal(o8, o16[:9])
        np.testing.assert_array_equal(t8, t16)
        np.testing.assert_array_equal(a8, a16[:8])
        np.testing.assert_array_equal(a.prev, b.prev)


def test_simulated_dialogue_equals_teacher_forced():
    """No user input: the user's slots are the model's own draws. The stream's 16 audio
    logits match a teacher-forced pass over the realised sequence, and every own token is
    its argmax once its stream has started (user slots follow the audio start rule)."""
    w = generate_weights(SIM, seed=0, threads=1)
    m = Oracle(SIM, w)
    S = 10
    sess = Session(m)
    outs, realised = [], []
    for s in range(S):
        own, lt, la = sess.step(None)
        outs.append((own, lt, la))
        realised.append(own.copy())
        np.testing.assert_array_equal(sess.prev, own)
    _, la_tf, _ = m.forward_teacher_forced(np.array(realised))
    for s, (own, lt, la) in enumerate(outs):
        assert _rel(la, la_tf[s]) < 1e-12
        for j in range(16):
            acoustic = j % 8 != 0
            pad = s < SIM.delay and acoustic
            assert own[1 + j] == (SIM.pad_audio if pad else np.argmax(la_tf[s, j]))
    with pytest.raises(ValueError):
        Session(Oracle(MICRO, generate_weights(MICRO, seed=0, threads=1))).step(None)


def test_sixteen_index_weights():
    from synth import param_count, weight_specs
    extra = param_count(SIM) - param_count(MICRO)
    per_index = sum(int(np.prod(shape)) for name, shape, _ in weight_specs(SIM) if name.startswith("depth.8."))
    assert extra == 8 * per_index
    assert [n for n, _, _ in weight_specs(SIM) if n.endswith(".head")][-1] == "depth.15.head"
