"""Helpers shared by the GPU parity tests (oracle runs, comparisons)."""
import numpy as np

from oracle import Oracle, Session, delay_codes, joint_sequence, top2_margin
from synth import raw_frames

MARGIN = 0.05


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def user_model_order(cfg, b, n_frames, seed=0):
    return delay_codes(raw_frames(cfg, b, n_frames, seed)["user"], cfg.delay, cfg.pad_audio)


def prompt_V(cfg, b, n_frames, seed=0):
    fr = raw_frames(cfg, b, n_frames, seed)
    return joint_sequence(cfg, fr["text"], fr["moshi"], fr["user"])


def oracle_greedy(model: Oracle, user, n, prompt=None):
    """Oracle streaming: optional teacher-forced prompt V[P, 17], then n greedy frames.
    Returns list of (own tokens, text logits, audio logits) for the greedy frames."""
    sess = Session(model)
    if prompt is not None:
        for s in range(prompt.shape[0]):
            sess.step(prompt[s, 9:], force=prompt[s, :9])
    out = []
    P = 0 if prompt is None else prompt.shape[0]
    for s in range(n):
        out.append(sess.step(user[P + s]))
    return out


def compare_frame(cfg, pos, own, lt, la, tok, glt, gla, tol):
    """Token parity where the oracle's margin exceeds 0.05; returns (worst rel-L2, n checked, n total)."""
    worst = max(rel_l2(glt, lt), max(rel_l2(gla[j], la[j]) for j in range(cfg.n_q)))
    assert worst <= tol, f"frame at position {pos}: logits rel-L2 {worst:.3g} > {tol}"
    checked = total = 0
    total += 1
    if top2_margin(lt) > MARGIN:
        checked += 1
        assert tok[0] == own[0], (pos, "text", tok[0], own[0])
    for j in range(cfg.n_q):
        if j >= 1 and pos < cfg.delay:
            assert tok[1 + j] == cfg.pad_audio
            continue
        total += 1
        if top2_margin(la[j]) > MARGIN:
            checked += 1
            assert tok[1 + j] == own[1 + j], (pos, "codebook", j, tok[1 + j], own[1 + j])
    return worst, checked, total
