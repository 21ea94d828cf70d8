"""Benchmark of the RQ-Transformer frame step on one MI355X.

Default workload: the 7B-shape bf16 model at batch 1 -- a 375-frame random
prompt prefilled into the KV cache, then 250 greedy frames with new random user
codes every frame. Prints one JSON line (frames/s, ms per frame, roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample).

    python bench.py [--steps K] [--warmup W] [--config b1_7b|b8_7b_5min|tf_7b|b1_7b_q8|b1_7b_asr|b1_7b_tts|b1_7b_sampled|b1_7b_sim|mimi_rvq|mimi_transformer|seanet|mid_bf16|tiny]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 matrix-core peak of one MI355X
COUNTERS = os.path.join(ROOT, "profiles", "gemv_gate_up_b1_7b_counters.md")
KERNEL_SRC = os.path.join(ROOT, "full_duplex_speech_amd", "csrc", "kernels_decode.hip")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs, or None once the kernel source has changed."""
    import hashlib
    try:
        fields = dict(l.split(": ", 1) for l in open(COUNTERS).read().splitlines() if ": " in l and not l.startswith("|"))
        if fields.get("kernel_source_sha256", "").strip() != hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest():
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def tf_pass_flops(cfg, B, S):
    """Algorithmic floating-point operations of one teacher-forced pass over B x S frames: every
    linear map of the temporal and depth models, the text and depth heads, and causal attention
    over the S(S+1)/2 key-query pairs (QK^T and PV); the depth attention over <= 8 positions is
    negligible and not counted."""
    M = B * S
    d, F, dd, Fd = cfg.d_t, cfg.ffn_t, cfg.d_d, cfg.ffn_d
    temporal = 2.0 * M * cfg.n_layers_t * (4 * d * d + 3 * d * F)
    head = 2.0 * M * cfg.vocab_text * d
    attn = 4.0 * B * cfg.n_layers_t * d * S * (S + 1) / 2
    depth = 2.0 * M * cfg.n_q * (dd * d + cfg.n_layers_d * (4 * dd * dd + 3 * dd * Fd) + cfg.codebook * dd)
    return temporal + head + attn + depth


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def joint_prompt(fds, cfg, b, n_frames, seed=0):
    """Random codec frames -> model-order frames [n, 17] (acoustic delay applied by the
    library's helper; a text-audio delay shifts the later modality, pad first)."""
    from synth import raw_frames
    fr = raw_frames(cfg, b, n_frames, seed)
    V = np.empty((n_frames, 17), np.int32)
    V[:, 0] = fr["text"]
    V[:, 1:9] = fds.moshi_delay_codes(fr["moshi"], cfg.delay, cfg.pad_audio)
    V[:, 9:] = fds.moshi_delay_codes(fr["user"], cfg.delay, cfg.pad_audio)
    t0, a0 = max(cfg.text_delay, 0), max(-cfg.text_delay, 0)
    if t0:
        V[t0:, 0] = V[:-t0, 0].copy()
        V[:t0, 0] = cfg.pad_text
    if a0:
        V[a0:, 1:] = V[:-a0, 1:].copy()
        V[:a0, 1:] = cfg.pad_audio
    return V


def tts_words(cfg, b, n_words=4096):
    """Random words of 1-3 text ids (ids 0 and 1 stand for PAD and EPAD)."""
    rng = np.random.default_rng([11, b])
    return [list(rng.integers(2, cfg.vocab_text, size=int(rng.integers(1, 4)))) for _ in range(n_words)]


def cpu_baseline(cfg, weights, B, P, frames, prompts, users):
    """The oracle (float32) on the host: prefill untimed, then `frames` greedy frames
    of conversation 0 timed, in the configuration's streaming mode."""
    from oracle import Oracle, Session, TtsTextControl, dequantized_weights
    cores = len(os.sched_getaffinity(0))
    if cfg.dtype == "q8":  # the 8-bit model computes with the quantise-dequantise image of its linear maps
        weights = dequantized_weights(weights)
    m = Oracle(cfg, weights, dtype=np.float32)
    sess = Session(m)
    if cfg.temp_text or cfg.temp_audio:
        sess.set_sampling(cfg.temp_text, cfg.temp_audio, 2024)
    t0 = time.perf_counter()
    if P:
        z, _ = m.temporal(np.concatenate([m.initial_frame[None], prompts[0][:P - 1]]), 0, sess.cache)
        sess.pos = P
        sess.prev = prompts[0][P - 1].copy()
    t_prefill = time.perf_counter() - t0
    ctl = TtsTextControl(tts_words(cfg, 0), 0, 1, 0.65, 0.5) if cfg.mode == "tts" else None
    t0 = time.perf_counter()
    for i in range(frames):
        if cfg.mode == "asr":
            force = np.concatenate([[-1], prompts[0][P + i, 1:9]])
            sess.step(users[0][P + i], force=force, text_only=True)
        elif cfg.n_depth == 16:
            sess.step(None)
        else:
            sess.step(users[0][P + i], text_choice=ctl.choose if ctl else None)
    dt = time.perf_counter() - t0
    return {"value": round(frames / dt, 4), "unit": "frames/s", "cores": cores, "kind": "oracle",
            "sample": f"{frames} generated frames of one conversation at positions {P}..{P + frames - 1} "
                      f"(float32 NumPy oracle; prompt prefill {t_prefill:.1f} s untimed); "
                      f"a batch of {B} costs {B}x on the host",
            "ms_per_frame": round(dt * 1000 / frames, 2)}


def bench_rvq(args, torch, fds):
    """Mimi's split RVQ: encode (512 -> 256 projection, semantic VQ + 7-level acoustic
    RVQ over 2048 codewords) and decode (codeword sums, 256 -> 512) of 4 x 3750 latent
    frames, seeded random latents, projections and codebooks."""
    torch.cuda.set_device(0)
    M, DZ, DQ, Q, N = 15000, 512, 256, 8, 2048
    g = torch.Generator(device="cpu").manual_seed(0)
    z = torch.randn(M, DZ, generator=g).cuda()
    w_in = (torch.randn(DQ, DZ, generator=g) / DZ ** 0.5).cuda()
    w_out = (torch.randn(DZ, DQ, generator=g) / DQ ** 0.5).cuda()
    cb = (torch.randn(Q, N, DQ, generator=g) * 4 / DQ ** 0.5).cuda()
    codes = torch.empty(M, Q, dtype=torch.int32, device="cuda")
    zh = torch.empty(M, DZ, device="cuda")
    work = torch.empty(fds.moshi_rvq_work_bytes(M, DQ, Q, N), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        fds.moshi_rvq_encode(z, M, DZ, w_in, DQ, cb, Q, N, codes, work, stream)
        fds.moshi_rvq_decode(codes, M, cb, Q, N, DQ, w_out, DZ, zh, work, stream)

    K = args.steps or 20
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / K
    flops = 2.0 * M * DZ * DQ * 2 + Q * 2.0 * M * N * DQ  # projections + distances
    ach = flops / dt / 1e12
    cpu = None
    if args.cpu_frames != 0:
        from oracle.rvq import decode, encode
        n = 200
        zc, wi, wo, c = z[:n].cpu().numpy(), w_in.cpu().numpy(), w_out.cpu().numpy(), cb.cpu().numpy()
        t1 = time.perf_counter()
        cc, _ = encode(zc, wi, c)
        decode(cc, c, wo)
        ct = time.perf_counter() - t1
        cpu = {"value": round(n / ct, 2), "unit": "frames/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{n} latent frames encoded and decoded by the float64 NumPy oracle"}
    out = {
        "metric": "Mimi split-RVQ encode + decode latent frames/s", "value": round(M / dt, 1), "unit": "frames/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(dt * 1000, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded random latents, projections and codebooks)",
        "config": {"workload": "Mimi split RVQ, 4 x 3750 latent frames, 512 -> 256, 8 codebooks x 2048",
                   "config": "mimi_rvq", "frames": M},
        "roofline": {"bound": "alu", "achieved": round(ach, 2), "peak": 157.3, "unit": "TFLOP/s",
                     "frac": round(ach / 157.3, 4), "traffic": None,
                     "kernel": "whole encode + decode (k_linear_f32, k_rvq_level x 8, k_rvq_sum)",
                     "flops_per_step": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def mimi_tf_flops(B, S, n_layers=8, d=512, f=2048, window=250):
    """Algorithmic FLOP of the bottleneck Transformer: the four linear maps per layer and
    attention over each query's min(t + 1, window) keys (QK^T and PV)."""
    M = B * S
    linear = 2.0 * M * (4 * d * d + 2 * d * f)
    keys = sum(min(t + 1, window) for t in range(S)) * B
    attn = 4.0 * keys * d
    return n_layers * (linear + attn)


def bench_mimi_transformer(args, torch, fds):
    """Mimi's bottleneck Transformer (8 layers, width 512, 250-frame window) over 4 x 3750
    latent frames, float32, seeded random weights and latents."""
    from synth.mimi_inputs import latents, mimi_weights, pack
    torch.cuda.set_device(0)
    B, S, L, W = 4, 3750, 8, 250
    wts = mimi_weights(L, seed=0, scale=0.1)
    x0 = torch.from_numpy(latents(B, S, seed=0)).cuda()
    x = x0.clone()
    wd = torch.from_numpy(pack(wts, L)).cuda()
    work = torch.empty(fds.moshi_mimi_transformer_work_bytes(B, S), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        x.copy_(x0)
        fds.moshi_mimi_transformer(x, B, S, wd, L, W, work, stream)

    K = args.steps or 10
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / K
    flops = mimi_tf_flops(B, S, L, window=W)
    ach = flops / dt / 1e12
    cpu = None
    if args.cpu_frames != 0:
        from oracle.mimi_transformer import forward
        n = 250
        xs = x0[0, :n].cpu().numpy()
        t1 = time.perf_counter()
        forward(xs, wts, L, 8, W)
        ct = time.perf_counter() - t1
        cpu = {"value": round(n / ct, 2), "unit": "frames/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"the first {n} frames of one sequence through the float64 NumPy oracle"}
    out = {
        "metric": "Mimi bottleneck Transformer latent frames/s", "value": round(B * S / dt, 1), "unit": "frames/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(dt * 1000, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded random latents and weights)",
        "config": {"workload": "Mimi bottleneck Transformer, 8 layers x 512, 4 x 3750 frames, 250-frame window",
                   "config": "mimi_transformer", "frames": B * S},
        "roofline": {"bound": "alu", "achieved": round(ach, 2), "peak": 157.3, "unit": "TFLOP/s",
                     "frac": round(ach / 157.3, 4), "traffic": None,
                     "kernel": "whole pass (k_gemm_f32 x 4, k_window_attn, k_layer_norm x 2 per layer)",
                     "flops_per_step": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def seanet_flops(B, S):
    """Algorithmic FLOP of one SEANet encode + decode: 2 * C_in * C_out * k per output
    sample of a convolution, per input sample of a transposed one."""
    from synth.mimi_inputs import seanet_layers
    enc, dec = seanet_layers()
    total, T = 0.0, S * 1920
    t = T
    for name, kind, ci, co, k, st in enc:
        t_out = t // st
        total += 2.0 * ci * co * k * t_out
        t = t_out
    t = S
    for name, kind, ci, co, k, st in dec:
        if kind == "tconv":
            total += 2.0 * ci * co * k * t
            t *= st
        else:
            total += 2.0 * ci * co * k * t
    return B * total


def bench_seanet(args, torch, fds):
    """Mimi's SEANet encoder + decoder over 4 x 3750 frames (4 x 5 minutes of 24 kHz
    audio), float32, seeded weights and test signals."""
    from synth.mimi_inputs import audio, pack_seanet, seanet_weights
    torch.cuda.set_device(0)
    B, S = 4, 3750
    w = seanet_weights(seed=0)
    a = torch.from_numpy(audio(B, S * 1920, seed=0)).cuda()
    we = torch.from_numpy(pack_seanet(w, "enc")).cuda()
    wd = torch.from_numpy(pack_seanet(w, "dec")).cuda()
    lat = torch.empty((B, S, 512), device="cuda")
    out = torch.empty((B, S * 1920), device="cuda")
    work = torch.empty(fds.moshi_seanet_work_bytes(B, S), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        fds.moshi_seanet_encode(a, B, S, we, lat, work, stream)
        fds.moshi_seanet_decode(lat, B, S, wd, out, work, stream)

    K = args.steps or 3
    for _ in range(max(min(args.warmup, 2), 1)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / K
    flops = seanet_flops(B, S)
    ach = flops / dt / 1e12
    cpu = None
    if args.cpu_frames != 0:
        from oracle.seanet import decode, encode
        n = 4
        x = audio(1, n * 1920, seed=0)[0]
        t1 = time.perf_counter()
        decode(encode(x, w), w)
        ct = time.perf_counter() - t1
        cpu = {"value": round(n / ct, 2), "unit": "frames/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{n} frames ({n * 80} ms of audio) encoded and decoded by the float64 "
                                           f"NumPy oracle"}
    out_line = {
        "metric": "Mimi SEANet encode + decode frames/s (80 ms of 24 kHz audio per frame)",
        "value": round(B * S / dt, 1), "unit": "frames/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(dt * 1000, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded weights; sums of random sinusoids plus noise)",
        "config": {"workload": "Mimi SEANet encoder + decoder, 4 x 3750 frames (4 x 5 min at 24 kHz)",
                   "config": "seanet", "frames": B * S},
        "roofline": {"bound": "alu", "achieved": round(ach, 2), "peak": 157.3, "unit": "TFLOP/s",
                     "frac": round(ach / 157.3, 4), "traffic": None,
                     "kernel": "whole encode + decode (k_conv_tiled, k_tconv_phase_weights)", "flops_per_step": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out_line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="b1_7b")
    ap.add_argument("--cpu-frames", type=int, default=None, help="oracle frames timed on the host (0: skip)")
    ap.add_argument("--kernel-iters", type=int, default=320)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the frame step runs on a "
              f"single MI355X; see DESIGN.md for how it would shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    import full_duplex_speech_amd as fds
    from synth import config, generate_weights, param_count

    if args.config == "mimi_rvq":
        return bench_rvq(args, torch, fds)
    if args.config == "mimi_transformer":
        return bench_mimi_transformer(args, torch, fds)
    if args.config == "seanet":
        return bench_seanet(args, torch, fds)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = config(args.config)
    tf_mode = cfg.tf_frames > 0
    B = cfg.tf_batch if tf_mode else cfg.batch
    P = cfg.prompt_frames
    K = args.steps if args.steps is not None else (1 if tf_mode else cfg.gen_frames)
    W = args.warmup if not tf_mode else min(args.warmup, 1)
    cpu_frames = args.cpu_frames if args.cpu_frames is not None else (0 if tf_mode else (50 if cfg.d_t < 1024 else 6))

    t0 = time.perf_counter()
    weights = generate_weights(cfg, seed=0)
    log(f"weights: {param_count(cfg) / 1e9:.3f} B params generated in {time.perf_counter() - t0:.1f} s")
    max_tf = B * cfg.tf_frames if tf_mode else 0
    eng = fds.Moshi(cfg, max_batch=B, max_tf_tokens=max_tf, tts_max_tokens=16384 if cfg.mode == "tts" else 0)
    t0 = time.perf_counter()
    eng.load_weights(weights)
    log(f"weights uploaded in {time.perf_counter() - t0:.1f} s; workspace {eng.ws_bytes / 1e9:.2f} GB")
    ctx = eng.ctx

    if tf_mode:
        S = cfg.tf_frames
        V = np.stack([joint_prompt(fds, cfg, b, S) for b in range(B)])
        tok_dev = torch.from_numpy(V).cuda()
        torch.cuda.synchronize()
        loss = fds.moshi_loss()
        for _ in range(W):
            fds.moshi_forward_teacher_forced(ctx, tok_dev, B, S, fds.MOSHI_DEVICE_PTRS, None, None, loss)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            fds.moshi_forward_teacher_forced(ctx, tok_dev, B, S, fds.MOSHI_DEVICE_PTRS, None, None, loss)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        frames_per_step = B * S
        log(f"teacher-forced: ce_text {loss.ce_text:.4f} ce_audio {loss.ce_audio:.4f}")
        workload = {"workload": f"7B-shape teacher-forced scoring, {B} x {S} frames", "config": cfg.name,
                    "batch": B, "frames": S}
    else:
        n_total = P + K + W
        prompts = [joint_prompt(fds, cfg, b, n_total) for b in range(B)]
        users = [p[:, 9:] for p in prompts]
        user_dev = torch.from_numpy(np.stack([users[b][P:P + max(K, W)] for b in range(B)], axis=1).copy()).cuda()
        flags = fds.MOSHI_DEVICE_PTRS
        force_dev = [None] * max(K, W)
        # a simulated dialogue: the 16-index depth draws the user's codes, none are given
        user_in = [None if cfg.n_depth == 16 else user_dev[i] for i in range(max(K, W))]
        out_dev = torch.empty((max(K, W), B, 17 if cfg.n_depth == 16 else 9), dtype=torch.int32, device="cuda")
        if cfg.mode == "asr":
            # streaming ASR: Moshi's audio is forced from the input, the text is free, no depth
            f = np.stack([prompts[b][P:P + max(K, W)] for b in range(B)], axis=1)[..., :9].copy()
            f[..., 0] = -1
            force_all = torch.from_numpy(f).cuda()
            force_dev = [force_all[i] for i in range(max(K, W))]
            flags |= fds.MOSHI_STEP_TEXT_ONLY
        torch.cuda.synchronize()

        def prefill():
            eng.reset()
            if P:
                pr = np.ascontiguousarray(np.stack([p[:P] for p in prompts]))
                fds.moshi_forward_teacher_forced(ctx, pr, B, P, fds.MOSHI_TF_FILL_KV | fds.MOSHI_TF_SKIP_DEPTH)
            if cfg.temp_text or cfg.temp_audio:
                fds.moshi_set_sampling(ctx, cfg.temp_text, cfg.temp_audio, 2024)
            if cfg.mode == "tts":
                for b in range(B):
                    fds.moshi_tts_text(ctx, b, tts_words(cfg, b), 0, 1, 0.65, 0.5)

        t0 = time.perf_counter()
        prefill()
        log(f"prefill {B} x {P} frames in {time.perf_counter() - t0:.2f} s")
        for i in range(W):
            fds.moshi_step(ctx, B, user_in[i], force_dev[i], out_dev[i], None, None, flags)
        fds.moshi_sync(ctx)
        prefill()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            fds.moshi_step(ctx, B, user_in[i], force_dev[i], out_dev[i], None, None, flags)
        fds.moshi_sync(ctx)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        frames_per_step = B
        log(f"{K} steps of {B} frame(s): {dt * 1000 / K:.3f} ms/step; last tokens {out_dev[K - 1, 0].tolist()}")
        shape = "7B-shape, 8-bit block weights" if cfg.dtype == "q8" else "7B-shape"
        what = {"asr": "streaming ASR (text 2 s behind the audio, audio forced, depth skipped)",
                "tts": "streaming TTS (audio 2 s behind the text, in-kernel text control)"}.get(cfg.mode,
                                                                                              "streaming decode")
        if cfg.n_depth == 16:
            what = "simulated dialogue (16-index depth draws both speakers)"
        if cfg.temp_text or cfg.temp_audio:
            what += f" sampled at temperatures {cfg.temp_text} (text) / {cfg.temp_audio} (audio)"
        workload = {"workload": f"{shape} {what}, batch {B}, {P}-frame prompt then {K} generated frames"
                    if cfg.d_t == 4096 else f"{cfg.name} streaming decode, batch {B}, {P}-frame prompt then "
                    f"{K} greedy frames", "config": cfg.name, "batch": B, "prompt_frames": P, "frames": K}

    ms_per_step = dt * 1000 / K
    value = frames_per_step * K / dt

    # dominant kernel: the SwiGLU gate/up weight stream (the largest share of the frame's bytes);
    # in the teacher-forced pass the gate/up GEMM (the largest share of the pass's FLOPs)
    roofline = None
    if tf_mode:
        us, flops = fds.moshi_time_kernel(ctx, "tf_gate_up", B, 8)
        ach = flops / (us * 1e-6) / 1e12
        aus, aflops = fds.moshi_time_kernel(ctx, "tf_attn", B, 8)
        pass_flops = tf_pass_flops(cfg, B, cfg.tf_frames)
        pass_tflops = pass_flops / (ms_per_step * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "k_gemm_bf16 (gate/up GEMM + SiLU product, one temporal layer)",
                    "flops_per_launch": flops, "us_per_launch": round(us, 1),
                    "other_kernels": {"tf_attn": {"us": round(aus, 1),
                                                  "TFLOP/s": round(aflops / (aus * 1e-6) / 1e12, 1)}},
                    "pass_flops": pass_flops, "pass_tflops": round(pass_tflops, 1),
                    "pass_frac": round(pass_tflops / MFMA_PEAK_TFLOPS, 4)}
    else:
        us, nbytes = fds.moshi_time_kernel(ctx, "ffn_gate_up", B, args.kernel_iters)
        ach = nbytes / (us * 1e-6) / 1e9
        # the counters were taken on this kernel at this shape (7B, bf16, one conversation)
        traffic = measured_traffic() if (cfg.d_t == 4096 and cfg.dtype == "bf16" and B == 1) else None
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": ("k_gemv_q8" if cfg.dtype == "q8" else "k_gemv") +
                              " (RMSNorm + gate/up + SiLU product, one temporal layer)",
                    "bytes_per_launch": nbytes, "us_per_launch": round(us, 3)}
        others = {}
        for kname in ("qkv", "wo", "ffn_down", "text_head", "attn"):
            kus, kb = fds.moshi_time_kernel(ctx, kname, B, 64)
            others[kname] = {"us": round(kus, 2), "GB/s": round(kb / (kus * 1e-6) / 1e9, 1)}
        roofline["other_kernels"] = others
        # whole-frame algorithmic bytes: every weight once + K/V read at the mean context
        # (8-bit linear maps: one code byte plus 4 bytes of fp16 scale and min per 32 weights)
        esz = 2 if cfg.dtype in ("bf16", "q8") else 4
        lin_esz = 1.125 if cfg.dtype == "q8" else esz
        lin = param_count(cfg) - (cfg.vocab_text + 1 + 16 * (cfg.codebook + 1)) * cfg.d_t \
            - (cfg.vocab_text + 1 + (cfg.n_depth - 1) * (cfg.codebook + 1)) * cfg.d_d
        if cfg.mode == "asr":  # no depth: the temporal layers, the norms and the text head only
            lin = cfg.n_layers_t * (4 * cfg.d_t ** 2 + 3 * cfg.d_t * cfg.ffn_t + 2 * cfg.d_t) \
                + cfg.vocab_text * cfg.d_t + cfg.d_t
        mean_ctx = P + (K + 1) / 2
        kv = B * cfg.n_layers_t * 2 * cfg.d_t * esz * mean_ctx
        frame_bytes = lin * lin_esz + kv
        roofline["frame_bytes_per_step"] = frame_bytes
        roofline["frame_frac"] = round(frame_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    if args.calibrate_copy:
        # an elementwise kernel that reads 256 MiB and writes 256 MiB
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"calibration: elementwise add over {src.numel() * 4 / 2**20:.0f} MiB (read + write), 3 times")

    cpu = None
    if cpu_frames:
        log(f"cpu baseline: oracle float32, {cpu_frames} frames")
        cpu = cpu_baseline(cfg, weights, B, P, cpu_frames, prompts, users)

    out = {
        "metric": "RQ-Transformer frames/sec and ms/frame at batch 1 and 8 (7B shape, bf16)",
        "value": round(value, 3), "unit": "frames/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype if cfg.dtype in ("bf16", "q8") else "f32",
        "data": "synthetic (seeded random-init weights, uniform random tokens)",
        "config": workload, "roofline": roofline, "cpu_baseline": cpu,
        "host": {"cpu": platform.processor() or platform.machine(), "cores": len(os.sched_getaffinity(0))},
    }
    print(json.dumps(out), flush=True)
    eng.close()


if __name__ == "__main__":
    main()
