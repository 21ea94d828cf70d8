"""GPU parity of Mimi's bottleneck Transformer against oracle.mimi_transformer
(float64): ragged sequences longer than the 250-frame window, a one-frame window,
and a full-size run (8 layers, 4 x 3750 frames) checked on one sequence."""
import numpy as np
import pytest

from oracle.mimi_transformer import forward
from parity_util import rel_l2
from synth.mimi_inputs import latents, mimi_weights, pack

pytestmark = pytest.mark.gpu


def run(B, S, n_layers, window, scale, seed=0):
    import torch
    import full_duplex_speech_amd as fds
    w = mimi_weights(n_layers, seed=seed, scale=scale)
    x = latents(B, S, seed=seed)
    xd = torch.from_numpy(x.copy()).cuda()
    wd = torch.from_numpy(pack(w, n_layers)).cuda()
    work = torch.empty(max(fds.moshi_mimi_transformer_work_bytes(B, S), 4), dtype=torch.uint8, device="cuda")
    fds.moshi_mimi_transformer(xd, B, S, wd, n_layers, window, work)
    torch.cuda.synchronize()
    return w, x, xd.cpu().numpy()


@pytest.mark.parametrize("B,S,window", [(2, 300, 250), (1, 70, 1), (3, 33, 250)])
def test_mimi_transformer_small(B, S, window):
    w, x, y = run(B, S, 2, window, scale=0.5)
    for b in range(B):
        ref = forward(x[b], w, 2, 8, window)
        err = rel_l2(y[b] - x[b], ref - x[b])  # the layers' contribution
        assert err <= 1e-4, (b, err)
        assert rel_l2(y[b], ref) <= 1e-5
    print(f"B={B} S={S} window={window}: ok")


def test_mimi_transformer_full_size_one_sequence():
    B, S = 4, 3750
    w, x, y = run(B, S, 8, 250, scale=0.1, seed=1)
    ref = forward(x[B - 1], w, 8, 8, 250)
    err = rel_l2(y[B - 1] - x[B - 1], ref - x[B - 1])
    assert err <= 1e-4, err
    print(f"full size, sequence {B - 1}: contribution rel-L2 {err:.2e}")


def test_mimi_transformer_arguments():
    import torch
    import full_duplex_speech_amd as fds
    from full_duplex_speech_amd import MoshiError
    d = torch.empty(16, dtype=torch.uint8, device="cuda")
    fds.moshi_mimi_transformer(d, 0, 10, d, 8, 250, d)           # no frames: nothing to do
    with pytest.raises(MoshiError):
        fds.moshi_mimi_transformer(d, 1, 10, d, 8, 0, d)        # window must be >= 1
