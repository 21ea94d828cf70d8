"""Oracle pins for temperature sampling: the Philox4x64-10 generator against
NumPy's own Philox bit generator, the uniform and Gumbel transforms, the
Gumbel-max draw against softmax(l / T) frequencies, and the wiring of the
counters into streaming steps. All on the CPU."""
import numpy as np
import pytest

from oracle import Oracle, Session, joint_sequence
from oracle.sampling import gumbel, philox4x64, sample, scores, uniforms
from synth import config, generate_weights, raw_frames

MICRO = config("tiny", name="micro", d_t=64, n_layers_t=2, n_heads_t=4, ffn_t=96, ctx_max=32,
               d_d=32, n_layers_d=2, n_heads_d=2, ffn_d=48, vocab_text=50, codebook=64)


@pytest.mark.parametrize("key", [(0, 0), (7, 9), (0xFFFFFFFFFFFFFFFF, 0x123456789ABCDEF0)])
def test_philox_matches_numpy_bit_generator(key):
    """NumPy's Philox (4x64, 10 rounds) bumps its counter before each block, so its
    first block under counter c is the permutation of c + 1."""
    rng = np.random.default_rng(3)
    for _ in range(4):
        c = rng.integers(0, 2 ** 63, size=4, dtype=np.uint64)
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=c)
        ref = bg.random_raw(4)
        c1 = c.copy()
        c1[0] += np.uint64(1)
        np.testing.assert_array_equal(philox4x64(c1[None], key)[0], ref)


def test_uniform_transform():
    u = uniforms(4001, seed=5, position=3, conversation=1, slot=2)
    assert u.dtype == np.float32 and u.shape == (4001,)
    assert (u > 0).all() and (u < 1).all()
    k = u.astype(np.float64) * 2 ** 24
    np.testing.assert_array_equal(k, np.round(k))
    assert (np.round(k) % 2 == 1).all()                     # (2m + 1) * 2^-24
    assert abs(float(u.mean()) - 0.5) < 0.02
    # every counter field changes the stream
    for kw in ({"seed": 6}, {"position": 4}, {"conversation": 2}, {"slot": 3}):
        args = dict(seed=5, position=3, conversation=1, slot=2)
        args.update(kw)
        assert not np.array_equal(uniforms(64, **args), u[:64])
    # element i uses word i % 4 of block i // 4: a prefix does not depend on n
    np.testing.assert_array_equal(uniforms(10, 5, 3, 1, 2), u[:10])


def test_gumbel_closed_form():
    """G = -log(-log U): G(e^-1) = 0 and P(G <= x) = exp(-exp(-x))."""
    assert abs(float(gumbel(np.float32(np.exp(-1.0))))) < 1e-6
    u = uniforms(200000, seed=1, position=0, conversation=0, slot=0)
    g = gumbel(u).astype(np.float64)
    for x in (-1.0, 0.0, 1.0, 2.5):
        assert abs(np.mean(g <= x) - np.exp(-np.exp(-x))) < 4e-3
    assert abs(g.mean() - 0.5772156649) < 0.01              # Euler-Mascheroni


@pytest.mark.parametrize("T", [0.6, 0.8, 2.0])
def test_gumbel_max_draws_follow_softmax(T):
    """Draw frequencies over many positions match softmax(l / T) (chi-square)."""
    logits = np.array([0.3, -1.2, 1.1, 0.0, 0.7, -0.4], dtype=np.float32)
    p = np.exp(logits / T - np.max(logits / T))
    p /= p.sum()
    N = 30000
    counts = np.zeros(len(logits))
    for pos in range(N):
        counts[sample(logits, T, seed=11, position=pos)] += 1
    chi2 = float(((counts - N * p) ** 2 / (N * p)).sum())
    assert chi2 < 25.0  # 5 degrees of freedom: P(chi2 > 25) < 2e-4


def test_temperature_limits():
    logits = np.array([0.1, 2.0, -0.5, 1.0], dtype=np.float32)
    assert sample(logits, 0.0) == 1
    assert all(sample(logits, 1e-3, position=p) == 1 for p in range(200))
    with pytest.raises(ValueError):
        sample(logits, -1.0)
    tie = np.zeros(8, dtype=np.float32)
    assert sample(tie, 0.0) == 0                               # greedy ties: lowest index
    u = np.full(8, 0.5, dtype=np.float32)
    assert sample(tie, 1.0, u=u) == 0                          # equal scores: lowest index
    s = scores(logits, 0.5, uniforms(4, 0, 0, 0, 0))
    assert s.dtype == np.float32


def test_sampled_stream_equals_teacher_forced_draws():
    """Sampled streaming: each own token is the draw of oracle.sampling from the
    teacher-forced logits of the realised sequence, at counter (position, slot)."""
    w = generate_weights(MICRO, seed=0, threads=1)
    m = Oracle(MICRO, w)
    S = 10
    fr = raw_frames(MICRO, 0, S)
    V = joint_sequence(MICRO, fr["text"], fr["moshi"], fr["user"])
    sess = Session(m, conversation=3)
    sess.set_sampling(0.7, 0.8, seed=1234)
    realised, owns = [], []
    for s in range(S):
        own, _, _ = sess.step(V[s, 9:])
        owns.append(own)
        realised.append(np.concatenate([own, V[s, 9:]]))
    lt, la, _ = m.forward_teacher_forced(np.array(realised))
    greedy_differs = 0
    for s in range(S):
        assert owns[s][0] == sample(lt[s], 0.7, 1234, s, 3, 0)
        greedy_differs += int(owns[s][0] != np.argmax(lt[s]))
        for j in range(MICRO.n_q):
            want = MICRO.pad_audio if (j >= 1 and s < MICRO.delay) else sample(la[s, j], 0.8, 1234, s, 3, j + 1)
            assert owns[s][1 + j] == want
    assert greedy_differs > 0
