"""Oracle pins for Mimi's split residual vector quantiser. All on the CPU."""
import numpy as np
import pytest

from oracle.rvq import decode, encode, nearest


def test_nearest_matches_brute_force():
    rng = np.random.default_rng(0)
    r = rng.standard_normal((7, 5))
    c = rng.standard_normal((11, 5))
    got = nearest(r, c)
    for i in range(7):
        best, bi = None, None
        for k in range(11):
            d = 0.0
            for e in range(5):
                d += (float(r[i, e]) - float(c[k, e])) ** 2
            if best is None or d < best:
                best, bi = d, k
        assert got[i] == bi


def test_ties_take_the_lowest_index():
    c = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0], [0.0, 1.0]])
    r = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 0.5]])
    np.testing.assert_array_equal(nearest(r, c), [0, 1, 0])


def _scaled_codebooks(rng, Q=8, N=64, D=16):
    """Level q's codewords at scale 100^-q: greedy RVQ then recovers any sum of one
    codeword per acoustic level exactly."""
    return np.stack([rng.standard_normal((N, D)) * (100.0 ** -max(q - 1, 0)) for q in range(Q)])


def test_acoustic_rvq_recovers_a_sum_of_codewords():
    rng = np.random.default_rng(1)
    Q, N, D = 8, 64, 16
    cb = _scaled_codebooks(rng, Q, N, D)
    want = rng.integers(0, N, size=(20, Q - 1))
    x = sum(cb[q][want[:, q - 1]] for q in range(1, Q))
    codes, resid = encode(x, np.eye(D), cb)               # identity projection
    np.testing.assert_array_equal(codes[:, 1:], want)
    assert np.abs(resid).max() < 1e-12
    np.testing.assert_array_equal(codes[:, 0], nearest(x, cb[0]))


def test_residual_never_grows_with_a_zero_codeword():
    rng = np.random.default_rng(2)
    Q, N, D = 8, 32, 12
    cb = rng.standard_normal((Q, N, D)) * 0.5
    cb[:, 5] = 0.0
    x = rng.standard_normal((40, D))
    r = x.copy()
    for q in range(1, Q):
        idx = nearest(r, cb[q])
        new = r - cb[q][idx]
        assert (np.linalg.norm(new, axis=1) <= np.linalg.norm(r, axis=1) + 1e-12).all()
        r = new
    _, resid = encode(x, np.eye(D), cb)
    np.testing.assert_allclose(resid, r, atol=1e-12)


def test_split_branches_are_independent():
    """The semantic VQ and the acoustic RVQ both read the projected latent: changing
    one branch's codebooks leaves the other branch's codes unchanged."""
    rng = np.random.default_rng(3)
    Q, N, D, Z = 8, 32, 8, 24
    cb = rng.standard_normal((Q, N, D))
    w = rng.standard_normal((D, Z)) / np.sqrt(Z)
    z = rng.standard_normal((30, Z))
    codes, _ = encode(z, w, cb)
    cb2 = cb.copy()
    cb2[1:] = rng.standard_normal((Q - 1, N, D))
    codes2, _ = encode(z, w, cb2)
    np.testing.assert_array_equal(codes[:, 0], codes2[:, 0])
    cb3 = cb.copy()
    cb3[0] = rng.standard_normal((N, D))
    codes3, _ = encode(z, w, cb3)
    np.testing.assert_array_equal(codes[:, 1:], codes3[:, 1:])


def test_decode_sums_both_branches():
    """One-hot codebooks: codeword k of level q is (q + 1) e_k, so the decoded latent
    before the output projection has (q + 1) at each chosen position."""
    Q, N, D = 8, 6, 6
    cb = np.stack([np.eye(N, D) * (q + 1) for q in range(Q)])
    codes = np.array([[0, 1, 2, 3, 4, 5, 0, 1], [5, 5, 5, 5, 5, 5, 5, 5]], dtype=np.int32)
    y = decode(codes, cb, np.eye(D))
    want = np.zeros((2, D))
    for m in range(2):
        for q in range(Q):
            want[m, codes[m, q]] += q + 1
    np.testing.assert_allclose(y, want)
    w_out = np.arange(D * 3, dtype=float).reshape(3, D)   # output projection applied last
    np.testing.assert_allclose(decode(codes, cb, w_out), want @ w_out.T)
