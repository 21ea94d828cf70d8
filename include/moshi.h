/*
 * moshi.h -- C ABI of the MI355X (gfx950) RQ-Transformer frame-step library.
 *
 * The library runs Moshi's per-frame RQ-Transformer step and its teacher-forced
 * scoring pass on one GPU. Terms and equations refer to these web pages:
 *   [W] the Chinese walkthrough of the Moshi technical report on 139.9.1.231
 *       (sections "使用 RQ-Transformer 的分层自回归建模" with Fig. 3,
 *       "音频建模 / 声学延迟" with eq. 4, "多流建模", "内心独白",
 *       "Moshi的联合序列建模" with eq. 6 and Fig. 4, "训练损失",
 *       "Helium 文本语言模型 / 架构");
 *   [N] the notes page "Moshi: a Speech-Text Foundation Model for Real-Time
 *       Dialogue" (sections 3b, 3c, 3d and 4).
 *
 * Token layout ("model order"): every frame holds K = 2*n_q + 1 = 17 ids
 * (eq. 6 / Fig. 4 of [W]): slot 0 the text token (Inner Monologue), slots
 * 1..8 Moshi's codebooks (1 semantic, 2..8 acoustic, delayed by `delay`
 * frames), slots 9..16 the user's codebooks in the same delayed order. The pad
 * id of the text slot is vocab_text, of audio slots codebook; pad marks an
 * absent token (the initial frame, delayed codebooks before the first frame).
 *
 * Conventions for every call:
 *   - return 0 (MOSHI_OK) or a negative MOSHI_E* code; moshi_last_error()
 *     gives a message. On error the context's state is unchanged.
 *   - pointers are host memory unless the call's flags include
 *     MOSHI_DEVICE_PTRS; host buffers are read/written only during the call.
 *   - calls on one context are not thread-safe.
 *   - all GPU work runs on a stream owned by the context; when a caller
 *     stream was given to moshi_create, every call is ordered after the work
 *     already queued on it and the caller stream waits for the call's work.
 */
#ifndef MOSHI_H
#define MOSHI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOSHI_OK 0
#define MOSHI_EINVAL (-1)   /* bad config, shape, pointer or token id */
#define MOSHI_ECONTEXT (-2) /* the step would exceed ctx_max positions */
#define MOSHI_ENOMEM (-3)   /* workspace too small or no free KV page */
#define MOSHI_EHIP (-4)     /* HIP runtime error (message has the HIP string) */
#define MOSHI_ESTATE (-5)   /* call not valid in this state (e.g. no weights) */

/* weight precision (moshi_config.dtype) */
#define MOSHI_F32 0
#define MOSHI_BF16 1
#define MOSHI_Q8 2 /* linear maps in 8-bit blocks of 32 (asymmetric MinMax, float16 scale and min;
                      walkthrough section "压缩Moshi及其对语音质量的影响", "量化格式"), quantised at
                      upload from the bf16-rounded weights; embeddings bf16, norms fp32; max_batch 1 */

/* flags */
#define MOSHI_DEVICE_PTRS 1   /* all array arguments are device pointers; the call
                                 only enqueues work (see moshi_sync) */
#define MOSHI_TF_FILL_KV 2    /* teacher-forced: keep the KV cache and continue
                                 streaming at frame S+1 */
#define MOSHI_TF_SKIP_DEPTH 4 /* teacher-forced: temporal pass and text only */
#define MOSHI_STEP_TEXT_ONLY 8 /* moshi_step: skip the Depth Transformer (streaming ASR) */

/* Model and capacity description. Shapes follow [W] "使用 RQ-Transformer ..."
 * (Temporal Transformer with the Helium architecture, Depth Transformer with
 * one weight set per codebook index) and [N] 3b/3c. */
typedef struct moshi_config {
  int32_t d_t, n_layers_t, n_heads_t, ffn_t; /* temporal width, layers, heads, SwiGLU hidden */
  int32_t ctx_max;                           /* max positions per conversation */
  int32_t d_d, n_layers_d, n_heads_d, ffn_d; /* depth width, layers, heads, SwiGLU hidden */
  int32_t vocab_text;                        /* text vocabulary (pad id = vocab_text) */
  int32_t codebook;                          /* codebook size N_A (pad id = codebook) */
  int32_t n_q;                               /* codebooks per speaker; must be 8 */
  int32_t delay;                             /* acoustic delay tau, in frames (>= 0) */
  float rope_base, norm_eps;                 /* RoPE base, RMSNorm epsilon */
  int32_t dtype;                             /* MOSHI_F32, MOSHI_BF16 or MOSHI_Q8 weights */
  int32_t max_batch;                         /* conversations per context (1..8) */
  int32_t page_frames;                       /* KV page size in frames (64) */
  int32_t n_pages;                           /* KV pages in the pool; 0 = max_batch*ceil(ctx_max/page_frames) */
  int32_t max_tf_tokens;                     /* max B*S of moshi_forward_teacher_forced (0 = ctx_max*max_batch) */
  int32_t text_delay;     /* frames between the text and the audio streams ([W] "推导流式ASR和TTS",
                             appendix C): > 0 delays the text (streaming ASR, Fig. 8), < 0 delays
                             every audio stream (streaming TTS, Fig. 9), 0 is the dialogue layout;
                             |text_delay| < ctx_max */
  int32_t tts_max_tokens; /* capacity of the per-conversation TTS text (moshi_tts_text); 0 = none */
  int32_t n_depth;        /* depth indices: 0 or 8 = Moshi's codebooks; 16 = also the user's, after
                             Moshi's in the same frame ([W] inference paragraph after Fig. 4: the
                             user stream modelled as an output gives simulated dialogues) */
} moshi_config;

/* One weight tensor handed to moshi_init_weights: float32, C-order. Names and
 * shapes ([out, in] for linear maps, [rows, dim] for embedding tables with the
 * pad row last):
 *   temporal.emb.{k}                k = 0..16, rows vocab_text+1 (k = 0) or codebook+1
 *   temporal.layers.{l}.{attn_norm,ffn_norm}            [d_t]
 *   temporal.layers.{l}.{wq,wk,wv,wo}                   [d_t, d_t]
 *   temporal.layers.{l}.{w_gate,w_up}                   [ffn_t, d_t]
 *   temporal.layers.{l}.w_down                          [d_t, ffn_t]
 *   temporal.out_norm [d_t], temporal.text_head [vocab_text, d_t]
 *   depth.{j}.in_proj [d_d, d_t], depth.{j}.emb rows vocab_text+1 (j = 0) or codebook+1
 *   depth.{j}.layers.{l}.* as for the temporal layers with d_d, ffn_d
 *   depth.{j}.out_norm [d_d], depth.{j}.head [codebook, d_d]       j = 0..7
 */
typedef struct moshi_tensor {
  const char* name;
  const float* data;
  int64_t numel;
  int32_t on_device; /* 1: data is a device pointer */
  int32_t reserved;
} moshi_tensor;

/* Cross-entropy of the teacher-forced pass ([W] "训练损失"; weights of [N] 4):
 * ce_text over the text slot; ce_per_cb[j] over Moshi's codebook j; ce_audio =
 * sum_j alpha_j ce_per_cb[j] / sum_j alpha_j with alpha = (100, 1, ..., 1);
 * ce_total = ce_text + ce_audio. Pad targets are excluded from every mean. */
typedef struct moshi_loss {
  double ce_text, ce_audio, ce_total;
  double ce_per_cb[8];
  int64_t n_text, n_audio;
} moshi_loss;

typedef struct moshi_ctx moshi_ctx;

/* Bytes of device workspace the context needs for `cfg` (0 if cfg is invalid). */
size_t moshi_workspace_bytes(const moshi_config* cfg);

/* Validate cfg; returns MOSHI_OK or MOSHI_EINVAL with a message in msg. */
int moshi_check_config(const moshi_config* cfg, char* msg, size_t msg_len);

/* Create a context on the current HIP device. `workspace` is caller-owned
 * device memory of at least moshi_workspace_bytes(cfg) bytes that outlives the
 * context; the library keeps weights, KV pages and activations in it.
 * `hip_stream` (may be NULL) is the caller's stream, see the conventions. */
int moshi_create(const moshi_config* cfg, void* hip_stream, void* workspace, size_t ws_bytes,
                 moshi_ctx** out);

/* Copy and repack weights (float32 in, converted to cfg.dtype). Every tensor
 * listed above must be given exactly once over one or more calls; the
 * context becomes usable when the last one has arrived. Synchronous. */
int moshi_init_weights(moshi_ctx* ctx, const moshi_tensor* tensors, int n);

/* Start conversation b afresh (b = -1: all): position 0, previous frame =
 * the all-pad initial frame V_0 ([W] "使用 RQ-Transformer ...": fixed initial
 * token), its KV pages returned to the pool, its TTS text control switched off. */
int moshi_reset(moshi_ctx* ctx, int b);

/* One frame for conversations 0..batch-1 ([W] Fig. 4 and the inference
 * paragraph after it; [N] 3d). Each conversation at position p consumes its
 * stored previous frame V_{s-1}, runs the Temporal Transformer one position,
 * takes the text token, then the Depth Transformer over Moshi's 8 codebooks.
 *   user_codes [batch][8]: the user's slots 9..16 of this frame (model order).
 *   force [batch][9] or NULL: Moshi's slots 0..8 to use instead of the
 *       model's own as depth inputs and as the stored frame (teacher forcing).
 *       An entry of -1 leaves that slot to the model, so one modality can be
 *       forced alone: the audio for streaming ASR ([W] appendix C, ASR mode),
 *       the text for TTS ([W] Fig. 9), or EPAD to make Moshi start speaking
 *       ([W] inference paragraph after Fig. 4).
 *   out_tokens [batch][9]: the model's own tokens: greedy (argmax, lowest index
 *       on ties) or temperature draws (moshi_set_sampling). A slot is pad before its stream starts: text while
 *       p < max(text_delay, 0), the semantic codebook while p < max(-text_delay, 0),
 *       acoustic codebooks 2..8 while p < max(-text_delay, 0) + delay.
 *       With a TTS text (moshi_tts_text) slot 0 is that control's choice.
 *   out_text_logits [batch][vocab_text], out_audio_logits [batch][8][codebook]:
 *       optional (NULL) float32 logits.
 *   With n_depth = 16: out_tokens is [batch][17] (slots 9..16: the model's draws
 *       of the user's codebooks), out_audio_logits [batch][16][codebook], and
 *       user_codes may be NULL: the user's slots of the stored frame are then the
 *       model's own draws (a simulated dialogue); given user codes drive the depth
 *       inputs of indices 9..15 and the stored frame. A text-only step needs
 *       user_codes and reports them in slots 9..16.
 *   flags: MOSHI_DEVICE_PTRS; MOSHI_STEP_TEXT_ONLY skips the Depth Transformer
 *       (streaming ASR discards the model's audio): slots 1..8 of out_tokens
 *       and of the stored frame are then the forced ids, or pad where force
 *       is NULL or -1, and out_audio_logits must be NULL.
 * Errors: MOSHI_ECONTEXT if some conversation is at ctx_max; MOSHI_EINVAL for
 * ids outside [0, pad] (force: [-1, pad]), with MOSHI_DEVICE_PTRS reported by
 * moshi_sync. */
int moshi_step(moshi_ctx* ctx, int32_t batch, const int32_t* user_codes, const int32_t* force,
               int32_t* out_tokens, float* out_text_logits, float* out_audio_logits, int32_t flags);

/* Temperature sampling of the own tokens of every later step (all conversations):
 * the text slot at temp_text, Moshi's codebooks at temp_audio; 0 = greedy (the
 * default). The pages sample at 0.6 (streaming TTS) and 0.8 (walkthrough, ASR/TTS
 * metrics paragraph after Table 9; audio-quality results of the quantisation
 * section); they fix no generator, so the draw is defined here:
 *   token = argmax_i (l_i / T + g_i) (lowest index on ties), g_i = -log(-log u_i),
 *   u_i = (2 (x >> 41) + 1) * 2^-24 with x word i % 4 of Philox4x64-10 (Salmon et
 *   al., SC'11) under key (seed, 0) at counter (i / 4, position, conversation,
 *   slot), slot 0 = text, 1..8 = codebooks; float32 arithmetic.
 * With a TTS text the PAD bonus is added to PAD's logit before the division by T.
 * Synchronises the context's stream. MOSHI_EINVAL for a negative or non-finite
 * temperature. */
int moshi_set_sampling(moshi_ctx* ctx, float temp_text, float temp_audio, uint64_t seed);

/* Zero-shot TTS text control of conversation `conv` ([W] appendix C, TTS mode and
 * Fig. 9). From the next step on, the text slot of that conversation is chosen
 * in the argmax kernel, per step:
 *   - inside a word (the next text token continues the word being fed): that
 *     token, without consulting the model;
 *   - otherwise the argmax of the text logits, with `bonus` added to the PAD logit
 *     while n_pad < target_pad_ratio * max(n_steps, 1) (float32; n_pad and n_steps
 *     count the PAD tokens and all tokens chosen so far). PAD or EPAD is kept;
 *     any other token is replaced by the first token of the next word, or by PAD
 *     once every word has been fed.
 * tokens [sum of word_lens]: the text ids of the words in speaking order, in
 * [0, vocab_text); word_lens [n_words] >= 1; pad_id, epad_id: the vocabulary's PAD
 * and EPAD ids; bonus >= 0. n_words = 0 switches the control off. A forced text
 * slot (force[b][0] >= 0) still overrides the choice for the frame it is given.
 * Host pointers; synchronises the context's stream. MOSHI_EINVAL for a bad
 * argument or more than tts_max_tokens tokens. */
int moshi_tts_text(moshi_ctx* ctx, int32_t conv, const int32_t* tokens, const int32_t* word_lens,
                   int32_t n_words, int32_t pad_id, int32_t epad_id, float target_pad_ratio, float bonus);

/* Teacher-forced pass over tokens [B][S][17] = V_1..V_S in model order
 * (inputs V_0..V_{S-1}, V_0 the pad frame) for conversations 0..B-1, which
 * must be at position 0. Outputs (each optional): text_logits [B][S][vocab_text],
 * audio_logits [B][S][8][codebook], loss (Moshi's 8 codebooks, also with
 * n_depth = 16, whose user indices are a streaming feature). With MOSHI_TF_FILL_KV the
 * conversations continue streaming at frame S+1; otherwise they are reset. */
int moshi_forward_teacher_forced(moshi_ctx* ctx, const int32_t* tokens, int32_t B, int32_t S,
                                 int32_t flags, float* text_logits, float* audio_logits,
                                 moshi_loss* loss);

/* Split residual vector quantiser of the Mimi codec (walkthrough sections
 * "量化率" and "使用分裂RVQ学习语义-声学token", Fig. 2; notes page 3a): the latent
 * z [M][dz] (dz = 512) is projected by w_in [dq][dz] (dq = 256); codebook 0 is a
 * plain VQ (semantic) and codebooks 1..Q-1 a residual VQ (acoustic), both applied
 * to the projected latent; the nearest codeword minimises the squared Euclidean
 * distance (float32, lowest index on ties). codebooks [Q][N][dq]; codes [M][Q].
 * Decoding sums the Q chosen codewords and projects by w_out [dz][dq] into
 * z_hat [M][dz]. All pointers are device pointers, float32 row-major; the calls
 * enqueue on hip_stream (NULL: the default stream) and need a caller-owned
 * device work buffer of moshi_rvq_work_bytes(M, dq, Q, N) bytes. dz and dq must
 * be multiples of 64 with dq <= 256, 2 <= Q <= 32. MOSHI_EINVAL for bad sizes or
 * null pointers (M = 0 does nothing), MOSHI_EHIP for a launch error. */
size_t moshi_rvq_work_bytes(int32_t M, int32_t dq, int32_t Q, int32_t N);
int moshi_rvq_encode(const float* z, int32_t M, int32_t dz, const float* w_in, int32_t dq, const float* codebooks,
                     int32_t Q, int32_t N, int32_t* codes, void* work, void* hip_stream);
int moshi_rvq_decode(const int32_t* codes, int32_t M, const float* codebooks, int32_t Q, int32_t N, int32_t dq,
                     const float* w_out, int32_t dz, float* z_hat, void* work, void* hip_stream);

/* Bottleneck Transformer of the Mimi codec (walkthrough section "基于 Transformer
 * 的瓶颈"; notes page 3a): n_layers pre-norm layers of width 512, 8 heads of 64,
 * MLP width 2048, applied in place to x [B][S][512] (B sequences of S frames,
 * positions from 0). Per layer:
 *   x += scale1 * Wo Attn(LN1(x));  x += scale2 * W2 GELU(W1 LN2(x))
 * LN: LayerNorm with gain and bias, eps 1e-5; GELU: x Phi(x) (erf); linear maps
 * without bias; Attn: RoPE (base 10000, consecutive pairs) on q and k, causal,
 * query t attending to keys t-window+1 .. t (the pages' 250 frames).
 * weights: float32, layers back to back, each [ln1_g 512][ln1_b 512][Wq 512x512]
 * [Wk][Wv][Wo][scale1 512][ln2_g 512][ln2_b 512][W1 2048x512][W2 512x2048]
 * [scale2 512], matrices [out][in] row-major. Device pointers, float32; enqueued
 * on hip_stream (NULL: default stream); work: a device buffer of
 * moshi_mimi_transformer_work_bytes(B, S) bytes. MOSHI_EINVAL for bad sizes or
 * null pointers (B*S = 0 does nothing), MOSHI_EHIP for a launch error. */
size_t moshi_mimi_transformer_work_bytes(int32_t B, int32_t S);
int moshi_mimi_transformer(float* x, int32_t B, int32_t S, const float* weights, int32_t n_layers, int32_t window,
                           void* work, void* hip_stream);

/* SEANet encoder / decoder of the Mimi codec (walkthrough, Mimi's baseline
 * architecture: causal residual convolution blocks with ELU, strides (4, 5, 6, 8)
 * and a final stride-2 convolution, mirrored by transposed convolutions; notes
 * page 3a). 24 kHz mono audio [B][S*1920] <-> latents [B][S][512] (12.5 frames/s).
 * Architecture (the pages give the strides; the rest is this library's reading):
 *   encoder: conv k7 1->64; per stride s in (4,5,6,8): residual unit
 *     x + conv_k1(ELU(conv_k3(ELU(x)))) (C -> C/2 -> C), then ELU + conv k=2s
 *     stride s (C -> 2C); ELU + conv k4 stride 2 (1024 -> 512).
 *   decoder: transposed conv k4 stride 2 (512 -> 1024); per stride in (8,6,5,4):
 *     ELU + transposed conv k=2s stride s (C -> C/2), residual unit; ELU + conv
 *     k7 (64 -> 1).
 * Causal: (k-1)+1-stride zeros on the left; transposed outputs past T*stride are
 * dropped. No biases (weight normalisation folded into the weights).
 * weights: float32, the encoder's (or the decoder's) convolutions back to back in
 * the order above; conv [C_out][C_in][k], transposed [C_in][C_out][k]. Device
 * pointers; enqueued on hip_stream (NULL: default); work: a device buffer of
 * moshi_seanet_work_bytes(B, S) bytes (288 floats per sample and sequence).
 * S * 1920 * 64 must fit in 31 bits. MOSHI_EINVAL for bad sizes or null pointers
 * (B*S = 0 does nothing), MOSHI_EHIP for a launch error. */
size_t moshi_seanet_work_bytes(int32_t B, int32_t S);
int moshi_seanet_encode(const float* audio, int32_t B, int32_t S, const float* weights, float* latents, void* work,
                        void* hip_stream);
int moshi_seanet_decode(const float* latents, int32_t B, int32_t S, const float* weights, float* audio, void* work,
                        void* hip_stream);

/* Kernels that moshi_time_kernel can time. */
#define MOSHI_KERNEL_QKV 0        /* RMSNorm + Wq|Wk|Wv + RoPE + KV append, one temporal layer */
#define MOSHI_KERNEL_WO 1         /* output projection + residual, one temporal layer */
#define MOSHI_KERNEL_FFN_GATE_UP 2 /* RMSNorm + gate/up + SiLU product, one temporal layer */
#define MOSHI_KERNEL_FFN_DOWN 3   /* down projection + residual, one temporal layer */
#define MOSHI_KERNEL_TEXT_HEAD 4  /* final RMSNorm + text head */
#define MOSHI_KERNEL_ATTN 5       /* causal decode attention over the filled cache, one layer */
#define MOSHI_KERNEL_TF_GATE_UP 6 /* teacher-forced gate/up GEMM + SiLU product, one temporal layer */
#define MOSHI_KERNEL_TF_ATTN 7    /* teacher-forced causal flash attention, one temporal layer */

/* Measurement: launch one kernel `iters` times on the context stream, cycling
 * over the temporal layers' weights (so that weights come from HBM as in a real
 * frame), between two HIP events; returns the mean time per launch in
 * microseconds and the algorithmic work of one launch in *bytes_per_launch:
 *   ids 0-5 (frame step, weight-streaming): bytes one launch must move
 *     (weights, plus activations, plus K/V for attention); they use the
 *     current activations and, for attention, the filled KV cache
 *     (position >= 1);
 *   ids 6-7 (teacher-forced pass, matrix cores): floating-point operations of
 *     one launch at the B x S shape of the last moshi_forward_teacher_forced
 *     call of this context, whose B `batch` must equal (attention counts the
 *     S(S+1)/2 causal pairs only).
 * The conversation state is left unchanged except for scratch activations. */
int moshi_time_kernel(moshi_ctx* ctx, int32_t kernel, int32_t batch, int32_t iters, float* avg_us,
                      double* bytes_per_launch);

/* MOSHI_Q8 models: copy the stored 8-bit form of linear tensor `name` (as named
 * for moshi_init_weights, [rows][cols]) to host buffers: codes[rows][cols],
 * and per block of 32 weights of a row scale[rows][cols/32] and
 * min[rows][cols/32] (float16 bit patterns); a weight is codes * scale + min.
 * MOSHI_EINVAL for an unknown, non-linear or not-yet-loaded tensor or a model
 * that is not MOSHI_Q8. */
int moshi_read_q8(moshi_ctx* ctx, const char* name, uint8_t* codes, uint16_t* scale, uint16_t* min);

/* Wait for queued work; reports device-side id errors of MOSHI_DEVICE_PTRS calls. */
int moshi_sync(moshi_ctx* ctx);

/* Current position (frames consumed) of conversation b, or a negative code. */
int moshi_position(const moshi_ctx* ctx, int b);

/* Host helper, [W] "音频建模 / 声学延迟" (eq. 4) and [N] 3c: codec frames
 * frames[T][8] -> model order out[T][8]: out[s][0] = frames[s][0],
 * out[s][q] = frames[s - tau][q] for q >= 1, pad where s - tau < 0. */
int moshi_delay_codes(const int32_t* frames, int32_t T, int32_t tau, int32_t pad, int32_t* out);

/* Host helper, inverse of moshi_delay_codes: model[T][8] -> out[T - tau][8]. */
int moshi_undelay_codes(const int32_t* model, int32_t T, int32_t tau, int32_t* out);

/* Last error message of ctx (or of the last failed moshi_create when ctx is NULL). */
const char* moshi_last_error(const moshi_ctx* ctx);

/* Release the context (not the caller's workspace). */
void moshi_destroy(moshi_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* MOSHI_H */
