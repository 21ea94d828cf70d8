"""GPU parity on the mid configuration (d=1024, 8 temporal layers, 32000-word text
vocabulary, 7B-shape depth), float32 and bf16 weights: a 375-frame prompt
prefilled into the KV cache, then 125 frames teacher-forced on the oracle's greedy
tokens; plus a 3750-frame context that spreads the decode attention over all of
its key splits."""
import numpy as np
import pytest

from oracle import Oracle, Session
from parity_util import compare_frame, prompt_V, rel_l2
from synth import config, generate_weights

pytestmark = pytest.mark.gpu

TOLS = {"mid_f32": 1e-4, "mid_bf16": 1e-2}


def oracle_prefilled(model, V, P):
    sess = Session(model)
    model.temporal(np.concatenate([model.initial_frame[None], V[:P - 1]]), 0, sess.cache)
    sess.pos = P
    sess.prev = V[P - 1].copy()
    return sess


def run_case(name, P, n, tol_scale=1.0):
    from full_duplex_speech_amd import Moshi
    cfg = config(name)
    tol = TOLS[name] * tol_scale
    w = generate_weights(cfg, seed=0)
    V = prompt_V(cfg, 0, P + n)
    model = Oracle(cfg, w)
    sess = oracle_prefilled(model, V, P)
    eng = Moshi(cfg, max_batch=1)
    eng.load_weights(w)
    eng.forward_teacher_forced(V[None, :P], fill_kv=True, skip_depth=True, logits=False, loss=False)
    worst, checked, total = 0.0, 0, 0
    for s in range(n):
        own, lt, la = sess.step(V[P + s, 9:])
        tok, glt, gla = eng.step(V[P + s, 9:][None], force=own[None], logits=True)
        wv, c, t = compare_frame(cfg, P + s, own, lt, la, tok[0], glt[0], gla[0], tol)
        worst, checked, total = max(worst, wv), checked + c, total + t
    eng.close()
    print(f"{name} P={P}: {n} frames, worst rel-L2 {worst:.2e}, tokens checked {checked}/{total}")
    return worst


@pytest.mark.parametrize("name", ["mid_f32", "mid_bf16"])
def test_mid_prompt_then_generate(name):
    cfg = config(name)
    run_case(name, cfg.prompt_frames, cfg.gen_frames)


def test_mid_long_context_all_splits():
    run_case("mid_bf16", 3750, 3)


def test_mid_teacher_forced_logits_and_loss():
    from full_duplex_speech_amd import Moshi
    from oracle import cross_entropy_loss
    cfg = config("mid_bf16")
    w = generate_weights(cfg, seed=0)
    B, S = 2, 24
    V = np.stack([prompt_V(cfg, b, S) for b in range(B)])
    model = Oracle(cfg, w)
    eng = Moshi(cfg, max_batch=B)
    eng.load_weights(w)
    lt, la, loss = eng.forward_teacher_forced(V)
    eng.close()
    rt, ra = zip(*[model.forward_teacher_forced(V[b])[:2] for b in range(B)])
    rt, ra = np.stack(rt), np.stack(ra)
    worst = max(rel_l2(lt[b, s], rt[b, s]) for b in range(B) for s in range(S))
    worst = max(worst, max(rel_l2(la[b, s, j], ra[b, s, j]) for b in range(B) for s in range(S) for j in range(8)))
    assert worst <= 1e-2
    ref = cross_entropy_loss(cfg, V, rt, ra)
    for k in ("ce_text", "ce_audio", "ce_total"):
        assert loss[k] == pytest.approx(ref[k], rel=1e-3)


def test_mid_bf16_teacher_forced_long_ragged():
    """Matrix-core teacher-forced pass over 2 x 300 frames (several 128-frame
    query tiles and 64-key tiles with a ragged tail), logits and loss against the
    oracle; then continue streaming after a FILL_KV pass."""
    from full_duplex_speech_amd import Moshi
    from oracle import cross_entropy_loss
    cfg = config("mid_bf16")
    w = generate_weights(cfg, seed=0)
    B, S = 2, 300
    V = np.stack([prompt_V(cfg, b, S) for b in range(B)])
    model = Oracle(cfg, w)
    eng = Moshi(cfg, max_batch=B)
    eng.load_weights(w)
    lt, la, loss = eng.forward_teacher_forced(V)
    refs = [model.forward_teacher_forced(V[b])[:2] for b in range(B)]
    rt = np.stack([r[0] for r in refs])
    ra = np.stack([r[1] for r in refs])
    worst = max(rel_l2(lt[b, s], rt[b, s]) for b in range(B) for s in range(S))
    worst = max(worst, max(rel_l2(la[b, s, j], ra[b, s, j]) for b in range(B) for s in range(0, S, 7) for j in range(8)))
    print(f"mid_bf16 teacher-forced 2x300: worst rel-L2 {worst:.2e}")
    assert worst <= 1e-2
    # argmax parity where the oracle's margin is clear
    from oracle import top2_margin
    mt = top2_margin(rt)
    ok = mt > 0.05
    assert (np.argmax(lt, -1)[ok] == np.argmax(rt, -1)[ok]).all()
    ref = cross_entropy_loss(cfg, V, rt, ra)
    for k in ("ce_text", "ce_audio", "ce_total"):
        assert loss[k] == pytest.approx(ref[k], rel=1e-3)
    eng.close()


@pytest.mark.parametrize("B", [2, 5])
def test_mid_bf16_batched_streaming(B):
    """Batch 2..8 runs the matrix-core GEMVs: RMSNorm statistics handed from the
    residual writers to the next normalising launch, and the down projection
    reading its fp16 input directly. Every conversation against its own oracle
    session, teacher-forced on the oracle's tokens."""
    from full_duplex_speech_amd import Moshi
    cfg = config("mid_bf16")
    w = generate_weights(cfg, seed=0)
    P, n = 40, 4
    Vs = [prompt_V(cfg, b, P + n) for b in range(B)]
    model = Oracle(cfg, w)
    refs = []
    for b in range(B):
        sess = oracle_prefilled(model, Vs[b], P)
        refs.append([sess.step(Vs[b][P + s, 9:]) for s in range(n)])
    eng = Moshi(cfg, max_batch=8)
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
            wv, _, _ = compare_frame(cfg, P + s, own, lt, la, tok[b], glt[b], gla[b], TOLS["mid_bf16"])
            worst = max(worst, wv)
    eng.close()
    print(f"mid_bf16 batch {B}: worst rel-L2 {worst:.2e}")


def test_mid_teacher_forced_kernel_timer():
    """moshi_time_kernel times the teacher-forced gate/up GEMM and flash attention
    at the shape of the last pass and reports their algorithmic FLOPs."""
    import full_duplex_speech_amd as fds
    from full_duplex_speech_amd import Moshi
    cfg = config("mid_bf16")
    w = generate_weights(cfg, seed=0)
    B, S = 2, 64
    V = np.stack([prompt_V(cfg, b, S) for b in range(B)])
    eng = Moshi(cfg, max_batch=B)
    eng.load_weights(w)
    eng.forward_teacher_forced(V, logits=False, loss=True)
    us, flops = fds.moshi_time_kernel(eng.ctx, "tf_gate_up", B, 2)
    assert us > 0 and flops == 2.0 * B * S * 2 * cfg.ffn_t * cfg.d_t
    us, flops = fds.moshi_time_kernel(eng.ctx, "tf_attn", B, 2)
    assert us > 0 and flops == 4.0 * B * cfg.d_t * S * (S + 1) / 2
    with pytest.raises(RuntimeError):
        fds.moshi_time_kernel(eng.ctx, "tf_gate_up", 1, 2)  # batch differs from the pass
    eng.close()
