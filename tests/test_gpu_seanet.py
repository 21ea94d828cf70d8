"""GPU parity of the SEANet encoder and decoder against oracle.seanet (float64):
a few frames of two sequences end to end, and the full size (4 x 3750 frames)
checked on the first frames of every sequence (both directions are causal, so a
prefix is exact)."""
import numpy as np
import pytest

from oracle.seanet import decode, encode
from parity_util import rel_l2
from synth.mimi_inputs import audio, pack_seanet, seanet_weights

pytestmark = pytest.mark.gpu


def run(B, S, seed=0):
    import torch
    import full_duplex_speech_amd as fds
    w = seanet_weights(seed=seed)
    a = audio(B, S * 1920, seed=seed)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ad, we, wd = dev(a), dev(pack_seanet(w, "enc")), dev(pack_seanet(w, "dec"))
    lat = torch.empty((B, S, 512), device="cuda")
    out = torch.empty((B, S * 1920), device="cuda")
    work = torch.empty(fds.moshi_seanet_work_bytes(B, S), dtype=torch.uint8, device="cuda")
    fds.moshi_seanet_encode(ad, B, S, we, lat, work)
    fds.moshi_seanet_decode(lat, B, S, wd, out, work)
    torch.cuda.synchronize()
    return w, a, lat.cpu().numpy(), out.cpu().numpy()


def test_seanet_small():
    B, S = 2, 3
    w, a, lat, out = run(B, S)
    for b in range(B):
        z = encode(a[b], w)
        assert rel_l2(lat[b], z) <= 1e-4, rel_l2(lat[b], z)
        y = decode(lat[b].astype(np.float64), w)   # the library's latents, decoded by the oracle
        assert rel_l2(out[b], y) <= 1e-4, rel_l2(out[b], y)
    print(f"latents {rel_l2(lat[0], encode(a[0], w)):.1e}")


def test_seanet_full_size_prefix():
    B, S, n = 4, 3750, 2
    w, a, lat, out = run(B, S, seed=1)
    for b in range(B):
        z = encode(a[b, :n * 1920], w)
        assert rel_l2(lat[b, :n], z) <= 1e-4
        y = decode(lat[b, :n].astype(np.float64), w)
        assert rel_l2(out[b, :n * 1920], y) <= 1e-4
    assert np.isfinite(lat).all() and np.isfinite(out).all()


def test_seanet_arguments():
    import torch
    import full_duplex_speech_amd as fds
    from full_duplex_speech_amd import MoshiError
    d = torch.empty(16, dtype=torch.uint8, device="cuda")
    fds.moshi_seanet_encode(d, 0, 5, d, d, d)                   # nothing to do
    with pytest.raises(MoshiError):
        fds.moshi_seanet_encode(d, 1, 1 << 20, d, d, d)         # too many samples
