"""GPU parity of the split residual vector quantiser against oracle.rvq.

Codes: at every level the oracle recomputes the residual from the library's own
earlier codes (float64) and checks the library's choice: it must be the nearest
codeword wherever the two least distances differ by more than the float32 bound,
and within that bound otherwise. Decoding is compared with the oracle's decoding
of the same codes."""
import numpy as np
import pytest

from oracle.rvq import decode

pytestmark = pytest.mark.gpu

DZ, DQ, Q, N = 512, 256, 8, 2048


def inputs(M, seed=0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, DZ)).astype(np.float32)
    w_in = (rng.standard_normal((DQ, DZ)) / np.sqrt(DZ)).astype(np.float32)
    w_out = (rng.standard_normal((DZ, DQ)) / np.sqrt(DQ)).astype(np.float32)
    scale = np.array([1.0] + [0.7 ** q for q in range(Q - 1)])
    cb = (rng.standard_normal((Q, N, DQ)) * scale[:, None, None] / np.sqrt(DQ) * 4).astype(np.float32)
    return z, w_in, w_out, cb


def run(M, seed=0):
    import torch
    import full_duplex_speech_amd as fds
    z, w_in, w_out, cb = inputs(M, seed)
    dev = lambda a: torch.from_numpy(a).cuda()
    zd, wi, wo, cbd = dev(z), dev(w_in), dev(w_out), dev(cb)
    codes = torch.empty((max(M, 1), Q), dtype=torch.int32, device="cuda")
    zh = torch.empty((max(M, 1), DZ), dtype=torch.float32, device="cuda")
    work = torch.empty(max(fds.moshi_rvq_work_bytes(M, DQ, Q, N), 4), dtype=torch.uint8, device="cuda")
    fds.moshi_rvq_encode(zd, M, DZ, wi, DQ, cbd, Q, N, codes, work)
    fds.moshi_rvq_decode(codes, M, cbd, Q, N, DQ, wo, DZ, zh, work)
    torch.cuda.synchronize()
    return (z, w_in, w_out, cb), codes.cpu().numpy()[:M], zh.cpu().numpy()[:M]


def check_codes(z, w_in, cb, codes, rows):
    exact = 0
    x = z[rows].astype(np.float64) @ w_in.astype(np.float64).T
    c64 = cb.astype(np.float64)
    for i, m in enumerate(rows):
        r = x[i].copy()
        for q in range(Q):
            src = x[i] if q == 0 else r
            d = ((c64[q] - src) ** 2).sum(axis=1)
            tol = 2e-5 * (float(src @ src) + float(np.max((c64[q] ** 2).sum(axis=1)))) + 1e-6
            g = int(codes[m, q])
            assert d[g] <= d.min() + tol, (m, q, g, d[g], d.min())
            two = np.sort(d)[:2]
            if two[1] - two[0] > tol:
                assert g == int(np.argmin(d)), (m, q)
                exact += 1
            if q:
                r = r - c64[q][g]
    return exact


@pytest.mark.parametrize("M", [1, 33, 1000])
def test_rvq_encode_decode(M):
    (z, w_in, w_out, cb), codes, zh = run(M)
    assert codes.min() >= 0 and codes.max() < N
    exact = check_codes(z, w_in, cb, codes, np.arange(M))
    ref = decode(codes, cb, w_out)
    rel = np.linalg.norm(zh - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5, rel
    print(f"M={M}: {exact} of {M * Q} codes checked exactly, decode rel-L2 {rel:.1e}")


def test_rvq_full_size_sampled():
    """4 x 3750 frames (four 5-minute streams): sampled rows checked against the oracle."""
    M = 15000
    (z, w_in, w_out, cb), codes, zh = run(M, seed=1)
    rows = np.random.default_rng(2).choice(M, size=120, replace=False)
    rows = np.concatenate([rows, [0, M - 1]])
    exact = check_codes(z, w_in, cb, codes, rows)
    ref = decode(codes[rows], cb, w_out)
    assert np.linalg.norm(zh[rows] - ref) / np.linalg.norm(ref) <= 1e-5
    assert exact > 0.9 * len(rows) * Q


def test_rvq_empty_and_bad_shapes():
    import torch
    import full_duplex_speech_amd as fds
    from full_duplex_speech_amd import MoshiError
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    fds.moshi_rvq_encode(dummy, 0, DZ, dummy, DQ, dummy, Q, N, dummy, dummy)      # M = 0: nothing to do
    with pytest.raises(MoshiError):
        fds.moshi_rvq_encode(dummy, 4, DZ, dummy, 100, dummy, Q, N, dummy, dummy)  # dq not a multiple of 64
    with pytest.raises(MoshiError):
        fds.moshi_rvq_encode(dummy, 4, DZ, dummy, 512, dummy, Q, N, dummy, dummy)  # dq above 256
