// Internal interfaces between the host engine and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moshi {

constexpr int kMaxBatch = 8;
constexpr int kSlots = 9;     // Moshi's own slots per frame: text + 8 codebooks
constexpr int kStreams = 17;  // slots per frame
constexpr int kMaxPagesPerConv = 512;  // ctx_max / page_frames

// Location of one key/value vector in a paged cache. A page holds `pf`
// consecutive positions of one conversation for every layer, laid out
// [layer][k|v][head][pos_in_page][hd]. Without a page table page = b.
struct KvView {
  void* base;
  const int* page_table;  // [B][pt_stride] physical page per logical page, or null
  int pt_stride;
  long long page_stride;  // elements per page
  int pf;                 // positions per page
  int n_heads;
  int hd;
  __device__ __forceinline__ long long offset(int b, int layer, int kv, int head, int p) const {
    int page = page_table ? page_table[b * pt_stride + p / pf] : b;
    return (long long)page * page_stride +
           ((long long)((layer * 2 + kv) * n_heads + head) * pf + (p % pf)) * hd;
  }
};

enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_EMB = 2, EPI_SWIGLU = 3, EPI_QKV = 4 };

struct GemvArgs {
  const void* W;  // [N][K] row-major, float or bf16 bits
  int N, K;
  const float* x;  // [B][ldx]
  int ldx;
  const float* gain;  // RMSNorm gain of x, or null (no normalisation)
  float eps;
  float* y;  // [B][ldy]
  int ldy;
  // EPI_QKV
  const int* pos;  // [B] positions, or null -> pos_const
  int pos_const;
  const float* rope;  // [positions][hd/2][cos, sin]
  int hd, d;          // head dim and model dim (q | k | v row boundaries)
  KvView kv;
  int kv_bf16;
  int layer;
  // 8-bit block weights (when set): W holds the codes q [N][K] (uint8) and
  // Wq8p the blocks' (scale | min << 16) float16 pairs [N][K/32]; w = q * scale + min
  const uint32_t* Wq8p;
  // EPI_SWIGLU: when set, also an fp16 copy of the outputs, [B][ldy]
  uint16_t* y16;
  // batched matrix-core path, RMSNorm statistics without re-reading x:
  // EPI_RESID / EPI_EMB write the sum of squares of each 16-row group of their
  // final outputs to stat_out[b * stat_out_ld + group]; a normalising launch
  // takes mean(x^2) from stat_in[b * stat_in_ld + 0 .. stat_in_n - 1], the
  // partials its producer wrote, added in a fixed order
  float* stat_out;
  int stat_out_ld;
  const float* stat_in;
  int stat_in_n, stat_in_ld;
  // batched matrix-core path: fp16 copy of x ([B][ldx], no normalisation)
  // read directly, for rows too long to stage in LDS
  const uint16_t* x16;
  // EPI_EMB: y = W x + emb[tok[b * tok_stride + tok_col]]
  const void* emb;
  const int* tok;
  int tok_stride, tok_col;
  int tok_rows;  // rows of emb (ids are clamped into range)
  // Output projection of one input vector (B = 1) with the attention finished
  // in the GEMV prologue, so that x is not read:
  //  - attn_q set: x = causal attention of the query heads attn_q (head h at
  //    h * hd) over keys 0..pos_const of the flat fp32 cache kv at `layer`,
  //    scores scaled by attn_scale (the depth model's at most 16 keys);
  //  - merge_part set: x = the merge of merge_ns key-range partials per head,
  //    [H][merge_ns][hd + 2] = (unnormalised o, running max, running sum)
  const float* attn_q;
  float attn_scale;
  const float* merge_part;
  int merge_ns;
};

struct AttnArgs {
  const float* q;  // [B][ldq], head h at h*hd
  int ldq;
  KvView kv;
  int layer;
  const int* pos;  // [B]: keys 0..pos[b]; null -> pos_const
  int pos_const;
  int split;       // unused
  float* part;     // [B][H][max_splits][hd + 2]
  int max_splits;  // key-range splits per (b, head); P / max_splits <= 512 keys
  int* counters;   // unused
  float* out;      // [B][ldo]
  int ldo;
  float scale;
};

struct EmbedArgs {
  const void* table;       // 17 tables back to back, rows of d elements
  const long long* row0;   // [17] first row of each table
  const int* rows;         // [17] rows of each table (pad row included)
  const int* frames;       // [B][17]
  float* h;                // [B][d]
  int d;
  int* err;
  float* stat_out;         // when set: sum of squares of h[b][256 j .. 256 j + 255] at [b * stat_ld + j]
  int stat_ld;
};

struct ArgmaxArgs {
  const float* logits;  // [B][ld]
  int n, ld;
  int slot;        // sub-stream 0..16 (counter of the sampling draw)
  int stride, col; // row stride and column of out_tok, cur_tok and force
  int start;       // the slot is pad_id while pos[b] < start (its stream has not begun)
  int pad_id;
  const int* pos;
  int* out_tok;    // [B][9] own tokens
  int* cur_tok;    // [B][9] tokens fed forward (forced or own)
  const int* force;      // [B][9]; an entry < 0 leaves the slot to the model
  const int* has_force;  // scalar flag
  // TTS text control of slot 0 (null: off): per conversation kTtsCtl words
  // {n tokens (0: off), cursor, n_pad, n_steps, pad id, epad id, target bits,
  // bonus bits} and the text, tokens [cap] and word-start flags [cap]
  int* tts_ctl;
  const int* tts_tok;
  const int* tts_start;
  int tts_cap;
  // temperature sampling: {text temperature, audio temperature} as float bits,
  // then the 64-bit seed (low, high word); temperature 0 = greedy
  const int* samp;
};
constexpr int kTtsCtl = 8;

struct AdvanceArgs {
  const int* cur_tok;  // [B][9]
  const int* force;      // [B][9], entries >= 0 used instead of cur_tok when *has_force
  const int* has_force;
  const int* user;     // [B][8]
  int* prev;           // [B][17]
  int* pos;            // [B]
  int* err;
  int pad_text, pad_audio;
  int text_only;  // no depth ran: slots 1..8 are forced or pad, also written to out_tok
  int* out_tok;   // [B][9]
  const int* user_cur;  // [B][8] user tokens of a 16-index depth (given or drawn), else null
};

struct CeRowsArgs {
  const float* text_logits;   // [B][ld_text]
  long long ld_text;
  const float* audio_logits;  // [B][ld_audio] = [B][8][codebook]
  long long ld_audio;
  const int* targets;         // [B][tgt_stride], slots 0..8
  int tgt_stride;
  int vocab_text, codebook;
  double* ce;                 // [B][S][9]
  int S, s;
};

enum TfEpi { TF_STORE_F32 = 0, TF_RESID = 1, TF_EMB = 2, TF_SWIGLU = 3, TF_QKV = 4 };

struct GemmArgs {
  const uint16_t* W;  // [N][K] fp16 (copy of the bf16 weight)
  const uint16_t* X;  // [M][ldx] fp16
  long long ldx;
  int M, N, K;
  float* Yf;          // float32 output / residual stream [M][ldy]
  uint16_t* Yb;       // bf16 output [M][ldy] (SwiGLU)
  long long ldy;
  // TF_EMB: Yf = acc + emb[tok[m * tok_stride]]
  const int* tok;
  long long tok_stride;
  int tok_rows;
  const uint16_t* emb;
  // TF_QKV
  int d, hd, S;
  int pos_const;      // >= 0: every row at this RoPE position (depth); < 0: position = m % S
  const float* rope;
  uint16_t* q;        // [M][ldq]
  long long ldq;
  KvView kv;
  int kv_paged;
  int layer;
  uint16_t* dk;       // flat K/V outputs [M][d] when !kv_paged
  uint16_t* dv;
};

struct FlashArgs {
  const uint16_t* q;  // [B*S][ldq]
  long long ldq;
  KvView kv;
  int layer;
  int S;
  float scale;
  uint16_t* out;      // [B*S][ldo]
  long long ldo;
};

struct DepthAttnArgs {
  const uint16_t* q;  // [8][M][d]
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;      // [M][d]
  long long M;
  int d, H, hd, j;
  float scale;
};

struct TfCeArgs {
  const float* text_logits;   // [M][vocab_text]
  const float* audio_logits;  // [M][8][codebook]
  const int* tokens;          // [M][17] targets V_s
  double* ce;                 // [M][9]
  int vocab_text, codebook;
};

// launchers (kernels_decode.hip)
void launch_gemv(const GemvArgs& a, int B, int epi, bool bf16, hipStream_t s);
void launch_attn_decode(const AttnArgs& a, int B, int H, int hd, bool kv_bf16, hipStream_t s);
// Attention followed by the output projection wo (EPI_RESID) at B = 1, with
// the attention's last step (the depth model's whole attention, or the merge
// of the temporal key-range splits) done in the projection's prologue. Returns
// false, launching nothing, when the shapes do not take the fused route.
bool launch_attn_wo(const AttnArgs& at, int B, int H, int hd, bool kv_bf16, GemvArgs wo, bool bf16, hipStream_t s);
void launch_embed(const EmbedArgs& a, int B, bool bf16, hipStream_t s);
void launch_argmax(const ArgmaxArgs& a, int B, hipStream_t s);
void launch_advance(const AdvanceArgs& a, int B, hipStream_t s);
// 8-bit blocks -> fp16 (w = q * scale + min), n elements from the start of a block
void launch_q8_to_f16(const uint8_t* q, const uint32_t* params, uint16_t* dst, long long n, hipStream_t s);
// bf16 -> fp16 element copy (round to nearest even; |x| > 65504 -> inf)
void launch_bf16_to_f16(const uint16_t* src, uint16_t* dst, long long n, hipStream_t s);
void launch_convert(const float* src, long long rows, int cols, void* dst, bool bf16, long long dst_row_mult,
                    long long dst_row_add, hipStream_t s);
// launchers (kernels_loss.hip)
void launch_ce_rows(const CeRowsArgs& a, int B, bool with_audio, hipStream_t s);
void launch_ce_reduce(const double* ce, long long n_rows, int n_slots, double* res, hipStream_t s);
void launch_rope_table(float* out, int P, int hd, double base, hipStream_t s);
// launchers (kernels_tf.hip)
void launch_gemm_bf16(const GemmArgs& g, int epi, hipStream_t s);
void launch_rmsnorm_f16(const float* x, long long ldx, const float* gain, float eps, int D, uint16_t* y,
                         long long ldy, long long rows, hipStream_t s);
void launch_tf_embed(const EmbedArgs& a, const int* tokens, long long M, int S, int pad_text, int pad_audio,
                     hipStream_t s);
void launch_flash_attn(const FlashArgs& f, int B, int H, int hd, hipStream_t s);
void launch_depth_attn(const DepthAttnArgs& a, hipStream_t s);
void launch_tf_ce(const TfCeArgs& a, long long M, bool with_audio, hipStream_t s);

}  // namespace moshi
