"""Plain CPU oracle of the Moshi RQ-Transformer frame step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this module. The HIP path shares no code with it; both only consume the seeded
inputs of the ``synth`` package.

Sources (web pages; cited by page and section, equation or figure):
  [W] the Chinese walkthrough of the Moshi technical report hosted on
      139.9.1.231 ("论文解读"), sections "Helium 文本语言模型 / 架构",
      "使用 RQ-Transformer 的分层自回归建模" (Fig. 3), "音频建模 / 声学延迟"
      (eq. 4), "多流建模", "内心独白", "Moshi的联合序列建模" (eq. 6, Fig. 4),
      "训练损失", "推导流式ASR和TTS", the inference paragraph after Fig. 4,
      and appendix C ("延迟文本语言模型作为zero-shot流式ASR和TTS", Figs. 8
      and 9);
  [N] the notes page "Moshi: a Speech-Text Foundation Model for Real-Time
      Dialogue", sections 3b (Helium), 3c (multi-stream generation) and 4
      (loss weighting);
  [E] the explainer post "语音多模态 Moshi：200ms 能抢话", sections 三 and 四.

Arithmetic is plain NumPy in the dtype given to ``Oracle`` (float64 by default;
float32 where memory forces it for 7B shapes). Nothing is blocked, fused or
reordered beyond the definitions below. Readings taken where the pages are
silent or garbled are marked READING.

Indexing: frames are 0-based here. Frame ``s`` (0-based) is frame s+1 of the
pages; the pages' deterministic initial frame V_0 is ``Oracle.initial_frame``.
Sub-streams are 0-based: 0 = text (Inner Monologue), 1 = Moshi semantic,
2..8 = Moshi acoustic, 9 = user semantic, 10..16 = user acoustic.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

# Loss weights of the 8 Moshi codebooks: semantic 100, acoustic 1 ([N] section 4,
# "Loss weighting"; [W] "训练损失").
ALPHA = np.array([100.0, 1, 1, 1, 1, 1, 1, 1])

# ---------------------------------------------------------------------------
# Token layout: acoustic delay and the joint sequence
# ---------------------------------------------------------------------------


def delay_codes(frames: np.ndarray, tau: int, pad: int) -> np.ndarray:
    """Place codec frames A[t, q] into the model's delayed order.

    [W] "音频建模 / 声学延迟" (eq. 4, whose formula the page lost) and [N] 3c:
    the semantic codebook (q = 0) is not delayed; acoustic codebooks q >= 1 lag
    it by ``tau`` steps. READING: model step s carries A[s, 0] and A[s - tau, q]
    for q >= 1; a source frame before the first one is ``pad``.
    """
    frames = np.asarray(frames)
    T, Q = frames.shape
    out = np.full((T, Q), pad, dtype=frames.dtype)
    for s in range(T):
        out[s, 0] = frames[s, 0]
        for q in range(1, Q):
            if s - tau >= 0:
                out[s, q] = frames[s - tau, q]
    return out


def undelay_codes(model: np.ndarray, tau: int) -> np.ndarray:
    """Inverse of ``delay_codes`` for the frames whose codebooks are all present."""
    model = np.asarray(model)
    T, Q = model.shape
    n = max(T - tau, 0)
    out = np.empty((n, Q), dtype=model.dtype)
    for t in range(n):
        out[t, 0] = model[t, 0]
        for q in range(1, Q):
            out[t, q] = model[t + tau, q]
    return out


def shift_stream(x: np.ndarray, n: int, pad: int) -> np.ndarray:
    """Delay a stream by n >= 0 steps along its first axis: step s carries
    x[s - n], and the first n steps (whose sources precede the first frame) are
    ``pad``."""
    x = np.asarray(x)
    out = np.full(x.shape, pad, dtype=x.dtype)
    for s in range(n, x.shape[0]):
        out[s] = x[s - n]
    return out


def n_depth(cfg) -> int:
    """Depth indices: Moshi's Q codebooks, or 2Q when the depth also predicts the
    user's codebooks ([W] inference paragraph after Fig. 4: modelling the user
    stream as an output lets the model generate both sides of a dialogue, used
    for offline evaluation). READING: index j >= Q predicts sub-stream j + 1, the
    user's codebook j - Q, with its own weights, after Moshi's Q in the same
    frame-local causal chain."""
    return 2 * cfg.n_q if int(getattr(cfg, "n_depth", cfg.n_q)) == 2 * cfg.n_q else cfg.n_q


def stream_starts(cfg) -> Tuple[int, int]:
    """First step at which the text stream and the audio streams carry frame 1.

    [W] "推导流式ASR和TTS" and appendix C: a delay between the text and the
    audio tokens selects the modality the model conditions on. ASR delays the
    text behind the audio (Fig. 8), TTS delays the audio behind the text
    (Fig. 9), both by 2 s (25 frames at 12.5 Hz) with acoustic delay 2.
    READING: ``cfg.text_delay`` is signed; a positive value delays the text
    stream by that many steps, a negative one delays every audio stream (Moshi's
    and the user's) by its magnitude, the acoustic delay applying on top.
    Returns (text_start, audio_start)."""
    d = int(getattr(cfg, "text_delay", 0))
    return max(d, 0), max(-d, 0)


def joint_sequence(cfg, text: np.ndarray, moshi: np.ndarray, user: np.ndarray) -> np.ndarray:
    """The joint sequence V[s, k] of [W] "Moshi的联合序列建模" (eq. 6, Fig. 4).

    K = 2Q + 1 sub-streams: the text token first ([W] "内心独白": text is the
    prefix of the semantic token), then Moshi's Q codebooks, then the user's Q
    codebooks, each audio stream delayed as in ``delay_codes`` ([W] "多流建模":
    the delay is applied to both audio streams before concatenation). With a
    text-audio delay (``stream_starts``) the delayed modality is shifted further.
    """
    T = len(text)
    t0, a0 = stream_starts(cfg)
    V = np.empty((T, cfg.n_streams), dtype=np.int32)
    V[:, 0] = shift_stream(text, t0, cfg.pad_text)
    V[:, 1:1 + cfg.n_q] = shift_stream(delay_codes(moshi, cfg.delay, cfg.pad_audio), a0, cfg.pad_audio)
    V[:, 1 + cfg.n_q:] = shift_stream(delay_codes(user, cfg.delay, cfg.pad_audio), a0, cfg.pad_audio)
    return V


# ---------------------------------------------------------------------------
# Helium building blocks ([W] "Helium 文本语言模型 / 架构"; [N] 3b)
# ---------------------------------------------------------------------------


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMS normalisation over the last axis: x / sqrt(mean(x^2) + eps) * g.

    [W] "Helium ... 架构": RMSNorm at the inputs of the attention block, the
    feed-forward block and the output linear layer.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding of x[T, H, hd] at integer positions pos[T].

    [W] "Helium ... 架构" uses RoPE. READING: consecutive pairs
    (x[2i], x[2i+1]) rotate by the angle pos * base^(-2i/hd).
    """
    hd = x.shape[-1]
    i = np.arange(hd // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]  # [T, hd/2]
    c = np.cos(ang)[:, None, :].astype(x.dtype)
    s = np.sin(ang)[:, None, :].astype(x.dtype)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Scaled dot-product attention with a causal mask.

    q[T, H, hd] sits at positions q_pos[T]; k, v[P, H, hd] hold positions
    0..P-1. Query t attends to keys 0..q_pos[t] with softmax(q.k / sqrt(hd))
    ([W] "Helium ... 架构": causal Transformer LM with FlashAttention, which
    computes exactly this softmax attention).
    """
    hd = q.shape[-1]
    scores = np.einsum("thd,phd->htp", q, k) / np.sqrt(hd).astype(q.dtype)
    P = k.shape[0]
    mask = np.arange(P)[None, :] > np.asarray(q_pos)[:, None]  # [T, P]
    scores = np.where(mask[None, :, :], -np.inf, scores)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("htp,phd->thd", w, v)


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x), the gate of Helium's gated linear unit."""
    return x / (1.0 + np.exp(-x))


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Difference between the largest and second-largest logit along the last axis."""
    part = np.partition(logits, -2, axis=-1)
    return part[..., -1] - part[..., -2]


# ---------------------------------------------------------------------------
# The model
# ---------------------------------------------------------------------------


class _Block:
    """Weights of one Helium block (pre-norm attention + SwiGLU, no biases)."""

    def __init__(self, w: Dict[str, np.ndarray], prefix: str, dt):
        g = lambda n: np.asarray(w[prefix + n], dtype=dt)  # noqa: E731
        self.attn_norm, self.ffn_norm = g("attn_norm"), g("ffn_norm")
        self.wq, self.wk, self.wv, self.wo = g("wq"), g("wk"), g("wv"), g("wo")
        self.w_gate, self.w_up, self.w_down = g("w_gate"), g("w_up"), g("w_down")


class Oracle:
    """RQ-Transformer of [W] "使用 RQ-Transformer 的分层自回归建模" (Fig. 3).

    A Temporal Transformer (Helium architecture) runs once per frame over time;
    a Depth Transformer (separate weights for every codebook index, [W] same
    section: per-index linear layers, projections and fully connected layers)
    then produces the codebooks of that frame one after another.
    """

    def __init__(self, cfg, weights: Dict[str, np.ndarray], dtype=np.float64):
        self.cfg = cfg
        self.dt = np.dtype(dtype)
        dt = self.dt
        g = lambda n: np.asarray(weights[n], dtype=dt)  # noqa: E731
        self.emb = [g(f"temporal.emb.{k}") for k in range(cfg.n_streams)]
        self.blocks = [_Block(weights, f"temporal.layers.{l}.", dt) for l in range(cfg.n_layers_t)]
        self.out_norm = g("temporal.out_norm")
        self.text_head = g("temporal.text_head")
        nd = n_depth(cfg)
        self.d_in = [g(f"depth.{j}.in_proj") for j in range(nd)]
        self.d_emb = [g(f"depth.{j}.emb") for j in range(nd)]
        self.d_blocks = [[_Block(weights, f"depth.{j}.layers.{l}.", dt) for l in range(cfg.n_layers_d)]
                         for j in range(nd)]
        self.d_out_norm = [g(f"depth.{j}.out_norm") for j in range(nd)]
        self.d_head = [g(f"depth.{j}.head") for j in range(nd)]

    # -- frame layout ---------------------------------------------------------
    @property
    def initial_frame(self) -> np.ndarray:
        """V_0: the deterministic initial frame ([W] "使用 RQ-Transformer ..." sets
        U_0 = 0 as a fixed initial token). READING: every sub-stream holds its pad id."""
        cfg = self.cfg
        f = np.full(cfg.n_streams, cfg.pad_audio, dtype=np.int32)
        f[0] = cfg.pad_text
        return f

    def embed(self, frames: np.ndarray) -> np.ndarray:
        """Temporal input: the sum over the K sub-streams of their learnt embedding
        rows ([W] "使用 RQ-Transformer ...": the input at step s is the sum of K
        learnt embedding tables of V_{s-1}). frames[T, K] -> [T, d_t]."""
        x = np.zeros((frames.shape[0], self.cfg.d_t), dtype=self.dt)
        for k in range(self.cfg.n_streams):
            x += self.emb[k][frames[:, k]]
        return x

    # -- one Helium block over T new positions with a KV cache ----------------
    def _block(self, b: _Block, h: np.ndarray, pos: np.ndarray, n_heads: int,
               cache: List[np.ndarray]) -> np.ndarray:
        """h <- h + W_o Attn(RMSNorm(h)); h <- h + W_down(SiLU(W_gate n) * W_up n), n = RMSNorm(h).

        [W] "Helium ... 架构"; [N] 3b. ``cache`` = [K, V] arrays of shape
        [P, H, hd] holding earlier positions 0..P-1; the new keys and values
        are appended and the queries attend causally.
        """
        cfg = self.cfg
        T, d = h.shape
        hd = d // n_heads
        n = rms_norm(h, b.attn_norm, cfg.norm_eps)
        q = (n @ b.wq.T).reshape(T, n_heads, hd)
        k = (n @ b.wk.T).reshape(T, n_heads, hd)
        v = (n @ b.wv.T).reshape(T, n_heads, hd)
        q = rope(q, pos, cfg.rope_base)
        k = rope(k, pos, cfg.rope_base)
        cache[0] = np.concatenate([cache[0], k], axis=0)
        cache[1] = np.concatenate([cache[1], v], axis=0)
        a = causal_attention(q, cache[0], cache[1], pos).reshape(T, d)
        h = h + a @ b.wo.T
        n = rms_norm(h, b.ffn_norm, cfg.norm_eps)
        h = h + (silu(n @ b.w_gate.T) * (n @ b.w_up.T)) @ b.w_down.T
        return h

    def new_temporal_cache(self) -> List[List[np.ndarray]]:
        cfg = self.cfg
        hd = cfg.d_t // cfg.n_heads_t
        e = np.zeros((0, cfg.n_heads_t, hd), dtype=self.dt)
        return [[e, e] for _ in range(cfg.n_layers_t)]

    def temporal(self, frames: np.ndarray, pos0: int, cache) -> Tuple[np.ndarray, np.ndarray]:
        """Temporal Transformer over input frames[T, K] at positions pos0..pos0+T-1.

        Returns z[T, d_t] (the context vector: the final RMSNorm output, READING
        of [W] "Helium ... 架构" which puts RMSNorm before the output linear)
        and the text logits l_{s,1} = Lin(z_s) ([W] "使用 RQ-Transformer ...").
        """
        T = frames.shape[0]
        pos = np.arange(pos0, pos0 + T)
        h = self.embed(frames)
        for l, b in enumerate(self.blocks):
            h = self._block(b, h, pos, self.cfg.n_heads_t, cache[l])
        z = rms_norm(h, self.out_norm, self.cfg.norm_eps)
        return z, z @ self.text_head.T

    # -- Depth Transformer ----------------------------------------------------
    def new_depth_cache(self, N: int) -> List[List[np.ndarray]]:
        cfg = self.cfg
        hd = cfg.d_d // cfg.n_heads_d
        e = np.zeros((N, 0, cfg.n_heads_d, hd), dtype=self.dt)
        return [[e, e] for _ in range(cfg.n_layers_d)]

    def depth_position(self, j: int, z: np.ndarray, tok_in: np.ndarray, cache) -> np.ndarray:
        """Depth position j (0-based) for N independent frames: logits of codebook j.

        [W] "使用 RQ-Transformer ...": the Depth Transformer maps z_s and the
        earlier sub-streams V_{s,1..k-1} of the same frame to the logits of
        V_{s,k}; every index k has its own linear, projection and fully
        connected weights (Table 6 ablation). READINGS: the input at position j
        is W_in^j z_s + E_D^j[V_{s,j}] (the projected context plus a learnt
        embedding of the previous sub-stream's token), the blocks are Helium
        blocks (RoPE at position j) attending causally over positions 0..j of
        the same frame, and the head is W_head^j RMSNorm^j(h).
        z[N, d_t], tok_in[N] -> logits[N, codebook].
        """
        cfg = self.cfg
        N = z.shape[0]
        H = cfg.n_heads_d
        hd = cfg.d_d // H
        h = z @ self.d_in[j].T + self.d_emb[j][tok_in]
        for l, b in enumerate(self.d_blocks[j]):
            n = rms_norm(h, b.attn_norm, cfg.norm_eps)
            q = (n @ b.wq.T).reshape(N, 1, H, hd)
            k = (n @ b.wk.T).reshape(N, 1, H, hd)
            v = (n @ b.wv.T).reshape(N, 1, H, hd)
            q = rope(q.reshape(N, H, hd), np.full(N, j), cfg.rope_base).reshape(N, 1, H, hd)
            k = rope(k.reshape(N, H, hd), np.full(N, j), cfg.rope_base).reshape(N, 1, H, hd)
            cache[l][0] = np.concatenate([cache[l][0], k], axis=1)  # [N, j+1, H, hd]
            cache[l][1] = np.concatenate([cache[l][1], v], axis=1)
            a = np.empty((N, H, hd), dtype=self.dt)
            for i in range(N):  # each frame attends only to its own positions 0..j
                a[i] = causal_attention(q[i], cache[l][0][i], cache[l][1][i], np.array([j]))[0]
            h = h + a.reshape(N, cfg.d_d) @ b.wo.T
            n = rms_norm(h, b.ffn_norm, cfg.norm_eps)
            h = h + (silu(n @ b.w_gate.T) * (n @ b.w_up.T)) @ b.w_down.T
        return rms_norm(h, self.d_out_norm[j], cfg.norm_eps) @ self.d_head[j].T

    # -- teacher-forced scoring ----------------------------------------------
    def forward_teacher_forced(self, V: np.ndarray, depth: bool = True):
        """Parallel teacher-forced pass over one conversation V[S, K] (V_1..V_S).

        Inputs are V_0..V_{S-1}; outputs are the text logits [S, vocab_text]
        predicting V_{s,1} and the audio logits [S, n_q, codebook] predicting
        V_{s,2..n_q+1}, the depth inputs being the true V_{s,1..n_q}
        ([W] "训练损失": the model is trained on the joint sequence of eq. 6
        with teacher forcing). Returns (text_logits, audio_logits, z).
        """
        S = V.shape[0]
        inp = np.concatenate([self.initial_frame[None, :], V[:-1]], axis=0)
        z, text_logits = self.temporal(inp, 0, self.new_temporal_cache())
        audio = None
        if depth:
            nd = n_depth(self.cfg)
            audio = np.empty((S, nd, self.cfg.codebook), dtype=self.dt)
            cache = self.new_depth_cache(S)
            for j in range(nd):
                audio[:, j] = self.depth_position(j, z, V[:, j], cache)
        return text_logits, audio, z


class Session:
    """Streaming inference, one frame per call ([W] "Moshi的联合序列建模", Fig. 4 and
    the inference paragraph after it: the model samples the text token and
    Moshi's codebooks; the user's codebooks are taken from the incoming audio
    and the model's predictions for them are not used). Decoding is greedy:
    argmax, the lowest index winning ties."""

    def __init__(self, model: Oracle, conversation: int = 0):
        self.m = model
        self.cache = model.new_temporal_cache()
        self.pos = 0
        self.prev = model.initial_frame.copy()
        self.conversation = conversation
        self.temps = (0.0, 0.0)
        self.seed = 0

    def set_sampling(self, temp_text: float, temp_audio: float, seed: int):
        """Temperature sampling of the own tokens (``oracle.sampling``); 0 = greedy."""
        self.temps = (float(temp_text), float(temp_audio))
        self.seed = int(seed)

    def pick(self, logits: np.ndarray, slot: int) -> int:
        """The own token of ``slot`` (0 text, 1..8 Moshi's codebooks) at this step."""
        from .sampling import sample
        t = self.temps[0] if slot == 0 else self.temps[1]
        return sample(logits, t, self.seed, self.pos, self.conversation, slot)

    def starts(self) -> np.ndarray:
        """Per own slot (text, semantic, 7 acoustic), the first frame whose source
        exists: earlier own tokens are pad (``stream_starts``, ``delay_codes``)."""
        cfg = self.m.cfg
        t0, a0 = stream_starts(cfg)
        audio = [a0] + [a0 + cfg.delay] * (cfg.n_q - 1)
        return np.array([t0] + audio * (n_depth(cfg) // cfg.n_q))

    def step(self, user_codes: np.ndarray, force: Optional[np.ndarray] = None, text_only: bool = False,
             text_choice=None):
        """Advance one frame. ``user_codes`` are the user's n_q sub-streams of this
        frame in model (delayed) order. ``force`` (optional, n_q + 1 ids) replaces
        the model's own tokens as depth inputs and as the stored frame; an entry
        of -1 leaves that slot to the model. This is the control the pages
        describe: ASR forces the audio and samples the text ([W] appendix C, ASR
        mode), TTS forces the text ([W] Fig. 9), and forcing EPAD makes Moshi
        start speaking ([W] inference paragraph after Fig. 4).

        ``text_only`` skips the Depth Transformer. Streaming ASR discards the
        model's audio predictions, so the depth is not run. The own audio tokens
        are then the forced ones, or pad where a slot is not forced, and the
        returned audio logits are None.

        ``text_choice`` (optional) replaces the draw of the text slot: it is
        called with the text logits and the sampler and returns the token (the
        TTS text control of ``oracle.tts_control``). Own tokens are greedy unless
        ``set_sampling`` chose temperatures.

        Returns (own tokens [n_q+1], text logits [vocab_text], audio logits
        [n_q, codebook]). Own tokens of a slot whose stream has not started are
        pad (``starts``).

        With a 16-index depth (``n_depth``) the depth goes on to the user's
        codebooks: own tokens and audio logits then have 2 n_q + 1 and 2 n_q
        rows. ``user_codes`` may be None: the user's slots of the stored frame
        are then the model's own draws (a simulated dialogue); given codes drive
        the depth inputs and the stored frame instead.
        """
        m, cfg = self.m, self.m.cfg
        if self.pos + 1 > cfg.ctx_max:
            raise ValueError("context overflow")
        st = self.starts()
        forced = (lambda k: force is not None and int(force[k]) >= 0)
        z, lt = m.temporal(self.prev[None, :], self.pos, self.cache)
        nd = n_depth(cfg)
        if user_codes is None and (nd == cfg.n_q or text_only):
            raise ValueError("user codes are needed unless the depth predicts them")
        own = np.empty(nd + 1, dtype=np.int32)
        pick_text = (lambda lg: self.pick(lg, 0))
        own[0] = int(text_choice(lt[0], pick_text)) if text_choice is not None else pick_text(lt[0])
        if self.pos < st[0]:
            own[0] = cfg.pad_text
        fed = own.copy()
        fed[0] = int(force[0]) if forced(0) else own[0]
        audio = None
        if text_only:
            for j in range(cfg.n_q):
                own[j + 1] = int(force[j + 1]) if forced(j + 1) else cfg.pad_audio
                fed[j + 1] = own[j + 1]
            for j in range(cfg.n_q, nd):
                own[j + 1] = fed[j + 1] = user_codes[j - cfg.n_q]
        else:
            audio = np.empty((nd, cfg.codebook), dtype=m.dt)
            dcache = m.new_depth_cache(1)
            tok = fed[0]
            for j in range(nd):
                audio[j] = m.depth_position(j, z, np.array([tok]), dcache)[0]
                t = self.pick(audio[j], j + 1)
                if self.pos < st[j + 1]:
                    t = cfg.pad_audio
                own[j + 1] = t
                if j < cfg.n_q:
                    fed[j + 1] = int(force[j + 1]) if forced(j + 1) else t
                else:
                    fed[j + 1] = t if user_codes is None else int(user_codes[j - cfg.n_q])
                tok = fed[j + 1]
        frame = np.empty(cfg.n_streams, dtype=np.int32)
        frame[:cfg.n_q + 1] = fed[:cfg.n_q + 1]
        frame[cfg.n_q + 1:] = fed[cfg.n_q + 1:] if nd > cfg.n_q else user_codes
        self.prev = frame
        self.pos += 1
        return own, lt[0], audio


def cross_entropy_loss(cfg, V: np.ndarray, text_logits: np.ndarray, audio_logits: np.ndarray) -> Dict:
    """Training loss of [W] "训练损失" with the weights of [N] section 4.

    V[B, S, K] are the targets, text_logits[B, S, vocab_text], audio_logits
    [B, S, n_q, codebook]. CE_text is the mean cross-entropy of the text
    sub-stream; CE_j the mean over codebook j of Moshi; CE_audio =
    sum_j alpha_j CE_j / sum_j alpha_j with alpha = 100 for the semantic and 1
    for the acoustic codebooks; the total gives text the same weight as all
    audio together. READING: pad targets (the absent delayed codebooks of the
    first frames) are left out of every mean.
    """
    def ce(logits, tgt, pad):
        keep = tgt != pad
        lg = logits[keep].astype(np.float64)
        t = tgt[keep]
        mx = lg.max(axis=-1, keepdims=True)
        lse = np.log(np.exp(lg - mx).sum(axis=-1)) + mx[:, 0]
        return float(np.mean(lse - lg[np.arange(len(t)), t])), int(keep.sum())

    ce_text, n_text = ce(text_logits.reshape(-1, cfg.vocab_text), V[..., 0].reshape(-1), cfg.pad_text)
    per_cb = []
    n_audio = 0
    for j in range(cfg.n_q):
        c, n = ce(audio_logits[:, :, j].reshape(-1, cfg.codebook), V[..., 1 + j].reshape(-1), cfg.pad_audio)
        per_cb.append(c)
        n_audio += n
    ce_audio = float(np.dot(ALPHA, per_cb) / ALPHA.sum())
    return {"ce_text": ce_text, "ce_audio": ce_audio, "ce_total": ce_text + ce_audio,
            "ce_per_cb": per_cb, "n_text": n_text, "n_audio": n_audio}
