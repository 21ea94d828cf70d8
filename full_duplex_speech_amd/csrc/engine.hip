// Host engine and C ABI (include/moshi.h): workspace plan, weight repack, KV
// page pool, frame-step sequencing with hipGraph replay, teacher-forced scoring.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <map>
#include <string>
#include <cmath>
#include <thread>
#include <utility>
#include <vector>

#include "../../include/moshi.h"
#include "moshi_internal.h"

using namespace moshi;

namespace {

struct Error {
  int code;
  std::string msg;
};

[[noreturn]] void fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  throw Error{code, buf};
}

#define HIPCHECK(expr)                                                                   \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) fail(MOSHI_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

std::string g_create_error;

struct LayerW {
  size_t wqkv, wo, wgu, wdown, attn_norm, ffn_norm;
};
struct DepthW {
  size_t in_proj, emb, out_norm, head;
  std::vector<LayerW> layers;
};
struct Dest {
  size_t off;      // byte offset of the destination region
  long long rows;  // source rows
  int cols;        // source columns
  long long mult, add;
  bool f32;        // stored as float32 regardless of dtype
  bool loaded;
  bool linear;     // a linear map (8-bit blocks in MOSHI_Q8 models)
};

struct Plan {
  bool bf = false;
  bool q8 = false;  // linear maps in 8-bit blocks (embeddings and KV bf16)
  int esz = 4;
  // 8-bit blocks: the codes of the bf16-layout element at byte offset o sit at
  // q8w + o/2, its block's parameters at q8p + o/16
  size_t q8w = 0, q8p = 0;
  size_t wbytes = 0;  // bytes of the weight region (offset 0)
  size_t total = 0;
  size_t take(size_t bytes) {
    size_t o = (total + 255) & ~(size_t)255;
    total = o + bytes;
    return o;
  }
  // weights
  size_t emb_t = 0;
  long long emb_row0[kStreams];
  int emb_rows[kStreams];
  std::vector<LayerW> lt;
  size_t out_norm = 0, text_head = 0;
  std::vector<DepthW> dj;
  // tables
  size_t meta_row0 = 0, meta_rows = 0, rope_t = 0, rope_d = 0;
  // KV
  size_t kv_pages = 0, page_table = 0, depth_kv = 0;
  long long page_elems = 0, depth_kv_elems = 0;
  int max_pages_conv = 0, n_pages = 0, max_splits = 0;
  // state (int32)
  size_t st_pos = 0, st_prev = 0, st_in = 0, st_out_tok = 0, st_cur_tok = 0, st_err = 0, st_cnt_t = 0,
         st_cnt_d = 0, st_end = 0;
  // TTS text control: per conversation kTtsCtl words of state (zeroed with the
  // step state: off), then the text and its word-start flags
  size_t tts_ctl = 0, tts_tok = 0, tts_start = 0;
  size_t st_samp = 0;  // sampling temperatures and seed (zeroed: greedy)
  size_t st_user_own = 0, st_user_cur = 0, st_user_given = 0;
  size_t st_user = 0, st_force = 0, st_has_force = 0;
  // activations (float32)
  size_t h = 0, q = 0, attn = 0, inter = 0, inter16 = 0, dinter16 = 0, part_t = 0, text_logits = 0;
  size_t hstat = 0, dstat = 0;  // per-16-row sums of squares of h / hd (batched steps)
  int hstat_ld = 0, dstat_ld = 0;
  size_t hd = 0, dq = 0, dattn = 0, dinter = 0, part_d = 0, audio_logits = 0;
  // teacher-forced
  size_t tf_tokens = 0, tf_ce = 0, tf_res = 0;
  long long tf_max = 0;
  bool tf_mfma = false;  // matrix-core teacher-forced pass (bf16 models)
  size_t w16 = 0;  // fp16 mirror of the weight region [0, meta_row0) for the matrix-core pass
  size_t tf_H = 0, tf_Xn = 0, tf_I = 0, tf_Q = 0, tf_O = 0, tf_text = 0;
  size_t tf_U = 0, tf_Xd = 0, tf_DQ = 0, tf_DK = 0, tf_DV = 0, tf_DO = 0, tf_DI = 0, tf_audio = 0;
  size_t staging = 0, staging_bytes = 0;
};

// depth indices: Moshi's 8 codebooks, or 16 when the depth also predicts the
// user's (simulated dialogues)
int depth_indices(const moshi_config& c) { return c.n_depth == 16 ? 16 : 8; }

int validate(const moshi_config& c, std::string& msg) {
  auto bad = [&](const char* m) {
    msg = m;
    return MOSHI_EINVAL;
  };
  if (c.d_t <= 0 || c.n_layers_t <= 0 || c.n_heads_t <= 0 || c.ffn_t <= 0 || c.ctx_max <= 0)
    return bad("temporal sizes must be positive");
  if (c.d_d <= 0 || c.n_layers_d <= 0 || c.n_heads_d <= 0 || c.ffn_d <= 0) return bad("depth sizes must be positive");
  if (c.d_t % c.n_heads_t || c.d_d % c.n_heads_d) return bad("model width must be a multiple of the head count");
  int hdt = c.d_t / c.n_heads_t, hdd = c.d_d / c.n_heads_d;
  if ((hdt != 32 && hdt != 64 && hdt != 128) || (hdd != 32 && hdd != 64 && hdd != 128))
    return bad("head dims must be 32, 64 or 128");
  if (c.d_t % 16 || c.d_d % 16) return bad("model widths must be multiples of 16");
  if (c.ffn_t % 8 || c.ffn_d % 8) return bad("SwiGLU widths must be multiples of 8");
  if (c.n_q != 8) return bad("n_q must be 8 (K = 17 sub-streams)");
  if (c.vocab_text < 2 || c.codebook < 2) return bad("vocabularies must have at least 2 entries");
  if (c.delay < 0) return bad("delay must be >= 0");
  if (c.text_delay <= -c.ctx_max || c.text_delay >= c.ctx_max) return bad("|text_delay| must be below ctx_max");
  if (c.tts_max_tokens < 0 || c.tts_max_tokens > (1 << 24)) return bad("tts_max_tokens must be in 0..2^24");
  if (c.n_depth != 0 && c.n_depth != 8 && c.n_depth != 16) return bad("n_depth must be 0, 8 or 16");
  if (!(c.rope_base > 0.f) || !(c.norm_eps > 0.f)) return bad("rope_base and norm_eps must be positive");
  if (c.dtype != MOSHI_F32 && c.dtype != MOSHI_BF16 && c.dtype != MOSHI_Q8)
    return bad("dtype must be MOSHI_F32, MOSHI_BF16 or MOSHI_Q8");
  if (c.dtype == MOSHI_Q8 && c.max_batch != 1) return bad("MOSHI_Q8 weights stream one conversation: max_batch must be 1");
  if (c.dtype == MOSHI_Q8 && (c.d_t % 32 || c.d_d % 32 || c.ffn_t % 32 || c.ffn_d % 32))
    return bad("MOSHI_Q8 needs every linear input width to be a multiple of 32");
  if (c.max_batch < 1 || c.max_batch > kMaxBatch) return bad("max_batch must be in 1..8");
  if (c.page_frames != 8 && c.page_frames != 16 && c.page_frames != 32 && c.page_frames != 64)
    return bad("page_frames must be 8, 16, 32 or 64");
  if (c.n_pages < 0 || c.max_tf_tokens < 0) return bad("n_pages and max_tf_tokens must be >= 0");
  if ((c.ctx_max + c.page_frames - 1) / c.page_frames > kMaxPagesPerConv)
    return bad("ctx_max / page_frames must be at most 512 pages");
  return MOSHI_OK;
}

Plan make_plan(const moshi_config& c) {
  Plan p;
  p.bf = c.dtype == MOSHI_BF16 || c.dtype == MOSHI_Q8;
  p.q8 = c.dtype == MOSHI_Q8;
  p.esz = p.bf ? 2 : 4;
  const size_t e = p.esz;
  const long long d = c.d_t, F = c.ffn_t, dd = c.d_d, Fd = c.ffn_d;
  long long rows = 0;
  for (int k = 0; k < kStreams; ++k) {
    p.emb_row0[k] = rows;
    p.emb_rows[k] = (k == 0 ? c.vocab_text : c.codebook) + 1;
    rows += p.emb_rows[k];
  }
  p.emb_t = p.take(rows * d * e);
  for (int l = 0; l < c.n_layers_t; ++l) {
    LayerW w;
    w.wqkv = p.take(3 * d * d * e);
    w.wo = p.take(d * d * e);
    w.wgu = p.take(2 * F * d * e);
    w.wdown = p.take(d * F * e);
    w.attn_norm = p.take(d * 4);
    w.ffn_norm = p.take(d * 4);
    p.lt.push_back(w);
  }
  p.out_norm = p.take(d * 4);
  p.text_head = p.take((long long)c.vocab_text * d * e);
  for (int j = 0; j < depth_indices(c); ++j) {
    DepthW w;
    w.in_proj = p.take(dd * d * e);
    w.emb = p.take((long long)((j == 0 ? c.vocab_text : c.codebook) + 1) * dd * e);
    for (int l = 0; l < c.n_layers_d; ++l) {
      LayerW x;
      x.wqkv = p.take(3 * dd * dd * e);
      x.wo = p.take(dd * dd * e);
      x.wgu = p.take(2 * Fd * dd * e);
      x.wdown = p.take(dd * Fd * e);
      x.attn_norm = p.take(dd * 4);
      x.ffn_norm = p.take(dd * 4);
      w.layers.push_back(x);
    }
    w.out_norm = p.take(dd * 4);
    w.head = p.take((long long)c.codebook * dd * e);
    p.dj.push_back(w);
  }
  p.wbytes = p.total;  // the weight region [0, wbytes)
  if (p.q8) {
    p.q8w = p.take(p.wbytes / 2);
    p.q8p = p.take(p.wbytes / 16);
  }
  p.meta_row0 = p.take(kStreams * 8);
  p.meta_rows = p.take(kStreams * 4);
  const int hdt = c.d_t / c.n_heads_t, hdd = c.d_d / c.n_heads_d;
  p.rope_t = p.take((size_t)c.ctx_max * hdt * 4);
  p.rope_d = p.take((size_t)depth_indices(c) * hdd * 4);
  // paged temporal KV (bf16 for bf16 models), flat depth KV (float32)
  p.max_pages_conv = (c.ctx_max + c.page_frames - 1) / c.page_frames;
  p.n_pages = c.n_pages ? c.n_pages : c.max_batch * p.max_pages_conv;
  p.page_elems = (long long)c.n_layers_t * 2 * c.d_t * c.page_frames;
  p.kv_pages = p.take((size_t)p.n_pages * p.page_elems * e);
  p.page_table = p.take((size_t)c.max_batch * p.max_pages_conv * 4);
  p.depth_kv_elems = (long long)c.n_layers_d * 2 * c.d_d * depth_indices(c);
  p.depth_kv = p.take((size_t)c.max_batch * p.depth_kv_elems * 4);
  // attention splits: every split covers at most 512 keys at full context
  p.max_splits = (c.ctx_max + 511) / 512;
  // state
  const int mb = c.max_batch;
  p.st_pos = p.take(mb * 4);
  p.st_prev = p.take(mb * kStreams * 4);
  p.st_in = p.take((mb * 8 + mb * kSlots + 1) * 4);
  p.st_user = p.st_in;
  p.st_force = p.st_in + mb * 8 * 4;
  p.st_has_force = p.st_force + mb * kSlots * 4;
  p.st_out_tok = p.take(mb * kSlots * 4);
  p.st_cur_tok = p.take(mb * kSlots * 4);
  p.st_err = p.take(4);
  p.st_cnt_t = p.take(mb * c.n_heads_t * 4);
  p.st_cnt_d = p.take(mb * c.n_heads_d * 4);
  if (c.tts_max_tokens) p.tts_ctl = p.take(mb * kTtsCtl * 4);
  p.st_samp = p.take(4 * 4);
  // 16-index depth: the user's own draws, the user tokens fed forward (given or
  // own), and whether this step's user codes were given
  p.st_user_own = p.take(mb * 8 * 4);
  p.st_user_cur = p.take(mb * 8 * 4);
  p.st_user_given = p.take(4);
  p.st_end = p.total;
  if (c.tts_max_tokens) {
    p.tts_tok = p.take((size_t)mb * c.tts_max_tokens * 4);
    p.tts_start = p.take((size_t)mb * c.tts_max_tokens * 4);
  }
  // activations
  p.h = p.take(mb * d * 4);
  p.q = p.take(mb * d * 4);
  p.attn = p.take(mb * d * 4);
  p.inter = p.take(mb * F * 4);
  p.inter16 = p.take(mb * F * 2);  // fp16 copy: input of the batched down projection
  p.hstat_ld = (int)((d + 15) / 16);
  p.hstat = p.take((size_t)mb * p.hstat_ld * 4);
  p.dstat_ld = (int)((dd + 15) / 16);
  p.dstat = p.take((size_t)mb * p.dstat_ld * 4);
  p.part_t = p.take((size_t)mb * c.n_heads_t * p.max_splits * (hdt + 2) * 4);
  p.text_logits = p.take((size_t)mb * c.vocab_text * 4);
  p.hd = p.take(mb * dd * 4);
  p.dq = p.take(mb * dd * 4);
  p.dattn = p.take(mb * dd * 4);
  p.dinter = p.take(mb * Fd * 4);
  p.dinter16 = p.take(mb * Fd * 2);
  p.part_d = p.take((size_t)mb * c.n_heads_d * (hdd + 2) * 4);
  p.audio_logits = p.take((size_t)mb * depth_indices(c) * c.codebook * 4);
  // teacher-forced
  const long long tf = c.max_tf_tokens ? c.max_tf_tokens : (long long)c.ctx_max * mb;
  p.tf_tokens = p.take((size_t)tf * kStreams * 4);
  p.tf_ce = p.take((size_t)tf * kSlots * 8);
  p.tf_res = p.take(32 * 8);
  p.tf_max = tf;
  // matrix-core pass: bf16 weights, GEMM K dims multiple of 32, head dims the
  // flash/depth attention kernels support
  p.tf_mfma = p.bf && d % 32 == 0 && F % 32 == 0 && dd % 32 == 0 && Fd % 32 == 0 && (hdt == 64 || hdt == 128) &&
              (hdd == 16 || hdd == 32 || hdd == 64);
  if (p.tf_mfma) {
    const size_t T = (size_t)tf;
    p.w16 = p.take(p.wbytes);
    p.tf_H = p.take(T * d * 4);
    p.tf_Xn = p.take(T * d * 2);
    p.tf_I = p.take(T * F * 2);
    p.tf_Q = p.take(T * d * 2);
    p.tf_O = p.take(T * d * 2);
    p.tf_text = p.take(T * c.vocab_text * 4);
    p.tf_U = p.take(T * c.n_q * dd * 4);
    p.tf_Xd = p.take(T * dd * 2);
    p.tf_DQ = p.take(T * c.n_q * dd * 2);
    p.tf_DK = p.take(T * c.n_q * dd * 2);
    p.tf_DV = p.take(T * c.n_q * dd * 2);
    p.tf_DO = p.take(T * dd * 2);
    p.tf_DI = p.take(T * Fd * 2);
    p.tf_audio = p.take(T * c.n_q * c.codebook * 4);
  }
  p.staging_bytes = 64ull << 20;
  p.staging = p.take(p.staging_bytes);
  p.total = (p.total + 255) & ~(size_t)255;
  return p;
}

}  // namespace

struct moshi_ctx {
  moshi_config cfg;
  Plan plan;
  char* ws = nullptr;
  hipStream_t stream = nullptr;      // owned
  hipStream_t caller = nullptr;      // optional caller stream
  hipEvent_t ev_in = nullptr, ev_out = nullptr;
  int device = 0;
  std::map<std::string, Dest> dests;
  size_t n_loaded = 0;
  bool ready = false;
  bool use_graph = true;
  bool tf_steps = false;  // teacher-forced pass as forced frame steps even for bf16 models
  int tf_B = 0, tf_S = 0;  // shape of the last matrix-core teacher-forced pass
  std::map<std::pair<int, int>, hipGraphExec_t> graphs;
  // host mirrors
  std::vector<int> pos_h;
  std::vector<std::vector<int>> pages;
  std::vector<int> free_pages;
  int* pinned = nullptr;  // staging: inputs block, outputs, page table mirror, constants
  size_t pinned_ints = 0;
  int* pin_in = nullptr;
  int* pin_out = nullptr;
  int* pin_pt = nullptr;
  int* pin_one = nullptr;
  int* pin_zero = nullptr;
  double* pin_res = nullptr;
  std::string err;

  template <typename T>
  T* at(size_t off) const {
    return (T*)(ws + off);
  }
};

namespace {

void add_dest(moshi_ctx* c, const std::string& name, size_t off, long long rows, int cols, long long mult = 1,
              long long add = 0, bool f32 = false) {
  static const char* kLinear[] = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "text_head", "in_proj", "head"};
  const std::string last = name.substr(name.rfind('.') + 1);
  bool lin = false;
  for (const char* l : kLinear) lin = lin || last == l;
  c->dests[name] = Dest{off, rows, cols, mult, add, f32, false, lin};
}

void build_dests(moshi_ctx* c) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  const size_t e = p.esz;
  const long long d = g.d_t, dd = g.d_d;
  for (int k = 0; k < kStreams; ++k)
    add_dest(c, "temporal.emb." + std::to_string(k), p.emb_t + p.emb_row0[k] * d * e, p.emb_rows[k], (int)d);
  auto layer = [&](const std::string& pre, const LayerW& w, long long D, long long F) {
    add_dest(c, pre + "attn_norm", w.attn_norm, 1, (int)D, 1, 0, true);
    add_dest(c, pre + "ffn_norm", w.ffn_norm, 1, (int)D, 1, 0, true);
    add_dest(c, pre + "wq", w.wqkv, D, (int)D);
    add_dest(c, pre + "wk", w.wqkv + D * D * e, D, (int)D);
    add_dest(c, pre + "wv", w.wqkv + 2 * D * D * e, D, (int)D);
    add_dest(c, pre + "wo", w.wo, D, (int)D);
    add_dest(c, pre + "w_gate", w.wgu, F, (int)D, 2, 0);  // gate rows at 2i
    add_dest(c, pre + "w_up", w.wgu, F, (int)D, 2, 1);    // up rows at 2i+1
    add_dest(c, pre + "w_down", w.wdown, D, (int)F);
  };
  for (int l = 0; l < g.n_layers_t; ++l) layer("temporal.layers." + std::to_string(l) + ".", p.lt[l], d, g.ffn_t);
  add_dest(c, "temporal.out_norm", p.out_norm, 1, (int)d, 1, 0, true);
  add_dest(c, "temporal.text_head", p.text_head, g.vocab_text, (int)d);
  for (int j = 0; j < depth_indices(g); ++j) {
    const std::string pre = "depth." + std::to_string(j) + ".";
    const DepthW& w = p.dj[j];
    add_dest(c, pre + "in_proj", w.in_proj, dd, (int)d);
    add_dest(c, pre + "emb", w.emb, (j == 0 ? g.vocab_text : g.codebook) + 1, (int)dd);
    for (int l = 0; l < g.n_layers_d; ++l) layer(pre + "layers." + std::to_string(l) + ".", w.layers[l], dd, g.ffn_d);
    add_dest(c, pre + "out_norm", w.out_norm, 1, (int)dd, 1, 0, true);
    add_dest(c, pre + "head", w.head, g.codebook, (int)dd);
  }
}

void order_in(moshi_ctx* c) {
  if (c->caller) {
    HIPCHECK(hipEventRecord(c->ev_in, c->caller));
    HIPCHECK(hipStreamWaitEvent(c->stream, c->ev_in, 0));
  }
}
void order_out(moshi_ctx* c) {
  if (c->caller) {
    HIPCHECK(hipEventRecord(c->ev_out, c->stream));
    HIPCHECK(hipStreamWaitEvent(c->caller, c->ev_out, 0));
  }
}

KvView temporal_kv(moshi_ctx* c) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  KvView v;
  v.base = c->ws + p.kv_pages;
  v.page_table = c->at<int>(p.page_table);
  v.pt_stride = p.max_pages_conv;
  v.page_stride = p.page_elems;
  v.pf = g.page_frames;
  v.n_heads = g.n_heads_t;
  v.hd = g.d_t / g.n_heads_t;
  return v;
}

KvView depth_kv(moshi_ctx* c) {
  const moshi_config& g = c->cfg;
  KvView v;
  v.base = c->ws + c->plan.depth_kv;
  v.page_table = nullptr;
  v.pt_stride = 0;
  v.page_stride = c->plan.depth_kv_elems;
  v.pf = depth_indices(g);
  v.n_heads = g.n_heads_d;
  v.hd = g.d_d / g.n_heads_d;
  return v;
}

// Argument builders of the frame's kernels (shared by the frame sequence and
// the kernel timer).
// weights of a streaming GEMV: the bf16/fp32 matrix at byte offset off, or its
// 8-bit codes and block parameters in MOSHI_Q8 models
void set_weights(moshi_ctx* c, GemvArgs& a, size_t off) {
  const Plan& p = c->plan;
  if (p.q8) {
    a.W = c->ws + p.q8w + off / 2;
    a.Wq8p = c->at<uint32_t>(p.q8p + off / 16);
  } else {
    a.W = c->ws + off;
  }
}

GemvArgs qkv_args(moshi_ctx* c, const LayerW& w, int layer, bool depth_model, int pos_const) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  const int D = depth_model ? g.d_d : g.d_t;
  GemvArgs a{};
  a.eps = g.norm_eps;
  set_weights(c, a, w.wqkv);
  a.N = 3 * D;
  a.K = D;
  a.x = c->at<float>(depth_model ? p.hd : p.h);
  a.ldx = D;
  a.gain = c->at<float>(w.attn_norm);
  a.y = c->at<float>(depth_model ? p.dq : p.q);
  a.ldy = D;
  a.pos = depth_model ? nullptr : c->at<int>(p.st_pos);
  a.pos_const = pos_const;
  a.rope = c->at<float>(depth_model ? p.rope_d : p.rope_t);
  a.hd = D / (depth_model ? g.n_heads_d : g.n_heads_t);
  a.d = D;
  a.kv = depth_model ? depth_kv(c) : temporal_kv(c);
  a.kv_bf16 = depth_model ? 0 : p.bf;
  a.layer = layer;
  return a;
}

AttnArgs attn_args(moshi_ctx* c, int layer, bool depth_model, int pos_const) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  const int D = depth_model ? g.d_d : g.d_t;
  const int hd = D / (depth_model ? g.n_heads_d : g.n_heads_t);
  AttnArgs at{};
  at.q = c->at<float>(depth_model ? p.dq : p.q);
  at.ldq = D;
  at.kv = depth_model ? depth_kv(c) : temporal_kv(c);
  at.layer = layer;
  at.pos = depth_model ? nullptr : c->at<int>(p.st_pos);
  at.pos_const = pos_const;
  at.split = depth_model ? depth_indices(g) : g.page_frames;
  at.part = c->at<float>(depth_model ? p.part_d : p.part_t);
  at.max_splits = depth_model ? 1 : p.max_splits;  // number of key-range splits
  at.counters = c->at<int>(depth_model ? p.st_cnt_d : p.st_cnt_t);
  at.out = c->at<float>(depth_model ? p.dattn : p.attn);
  at.ldo = D;
  at.scale = 1.0f / sqrtf((float)hd);
  return at;
}

GemvArgs wo_args(moshi_ctx* c, const LayerW& w, bool depth_model) {
  const Plan& p = c->plan;
  const int D = depth_model ? c->cfg.d_d : c->cfg.d_t;
  GemvArgs o{};
  set_weights(c, o, w.wo);
  o.N = D;
  o.K = D;
  o.x = c->at<float>(depth_model ? p.dattn : p.attn);
  o.ldx = D;
  o.y = c->at<float>(depth_model ? p.hd : p.h);
  o.ldy = D;
  return o;
}

GemvArgs gu_args(moshi_ctx* c, const LayerW& w, bool depth_model) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  const int D = depth_model ? g.d_d : g.d_t, F = depth_model ? g.ffn_d : g.ffn_t;
  GemvArgs f{};
  f.eps = g.norm_eps;
  set_weights(c, f, w.wgu);
  f.N = 2 * F;
  f.K = D;
  f.x = c->at<float>(depth_model ? p.hd : p.h);
  f.ldx = D;
  f.gain = c->at<float>(w.ffn_norm);
  f.y = c->at<float>(depth_model ? p.dinter : p.inter);
  f.y16 = c->at<uint16_t>(depth_model ? p.dinter16 : p.inter16);
  f.ldy = F;
  return f;
}

GemvArgs down_args(moshi_ctx* c, const LayerW& w, bool depth_model) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  const int D = depth_model ? g.d_d : g.d_t, F = depth_model ? g.ffn_d : g.ffn_t;
  GemvArgs dn{};
  set_weights(c, dn, w.wdown);
  dn.N = D;
  dn.K = F;
  dn.x = c->at<float>(depth_model ? p.dinter : p.inter);
  dn.x16 = c->at<uint16_t>(depth_model ? p.dinter16 : p.inter16);  // written by every SwiGLU epilogue
  dn.ldx = F;
  dn.y = c->at<float>(depth_model ? p.hd : p.h);
  dn.ldy = D;
  return dn;
}

GemvArgs text_head_args(moshi_ctx* c) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  GemvArgs a{};
  a.eps = g.norm_eps;
  set_weights(c, a, p.text_head);
  a.N = g.vocab_text;
  a.K = g.d_t;
  a.x = c->at<float>(p.h);
  a.ldx = g.d_t;
  a.gain = c->at<float>(p.out_norm);
  a.y = c->at<float>(p.text_logits);
  a.ldy = g.vocab_text;
  return a;
}

ArgmaxArgs argmax_args(moshi_ctx* c, int slot) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  ArgmaxArgs m{};
  if (slot == 0) {
    m.logits = c->at<float>(p.text_logits);
    m.n = g.vocab_text;
    m.ld = g.vocab_text;
  } else {
    m.logits = c->at<float>(p.audio_logits) + (long long)(slot - 1) * g.codebook;
    m.n = g.codebook;
    m.ld = depth_indices(g) * g.codebook;
  }
  m.slot = slot;
  // own slots are pad until their stream starts: the text after max(text_delay, 0)
  // frames, the audio after max(-text_delay, 0), the acoustic codebooks delay
  // later (the user's codebooks 9..16 like Moshi's 1..8)
  const int text_start = std::max(g.text_delay, 0), audio_start = std::max(-g.text_delay, 0);
  const int q = slot >= kSlots ? slot - kSlots + 1 : slot;
  m.start = slot == 0 ? text_start : (q == 1 ? audio_start : audio_start + g.delay);
  m.pad_id = slot == 0 ? g.vocab_text : g.codebook;
  m.samp = c->at<int>(p.st_samp);
  if (slot == 0 && g.tts_max_tokens) {
    m.tts_ctl = c->at<int>(p.tts_ctl);
    m.tts_tok = c->at<int>(p.tts_tok);
    m.tts_start = c->at<int>(p.tts_start);
    m.tts_cap = g.tts_max_tokens;
  }
  m.pos = c->at<int>(p.st_pos);
  if (slot < kSlots) {
    m.out_tok = c->at<int>(p.st_out_tok);
    m.cur_tok = c->at<int>(p.st_cur_tok);
    m.force = c->at<int>(p.st_force);
    m.has_force = c->at<int>(p.st_has_force);
    m.stride = kSlots;
    m.col = slot;
  } else {
    // the user's codebook slot - 9: given user codes act as forcing
    m.out_tok = c->at<int>(p.st_user_own);
    m.cur_tok = c->at<int>(p.st_user_cur);
    m.force = c->at<int>(p.st_user);
    m.has_force = c->at<int>(p.st_user_given);
    m.stride = 8;
    m.col = slot - kSlots;
  }
  return m;
}

// Enqueue one frame for conversations 0..B-1 (no host interaction).
// Batched bf16 steps (matrix-core GEMVs) pass the RMSNorm statistics of the
// residual streams from the kernel that writes them to the next normalising
// one instead of re-reading the vectors. Producers: the embedding (one partial
// per 256 features), residual GEMVs and the depth input projection (one per 16
// rows).
bool stats_on(moshi_ctx* c, int B) { return c->plan.bf && B >= 2; }
void stat_consume(moshi_ctx* c, GemvArgs& a, int B, bool depth_model, int n) {
  if (!stats_on(c, B)) return;
  const Plan& p = c->plan;
  a.stat_in = c->at<float>(depth_model ? p.dstat : p.hstat);
  a.stat_in_ld = depth_model ? p.dstat_ld : p.hstat_ld;
  a.stat_in_n = n;
}
void stat_produce(moshi_ctx* c, GemvArgs& a, int B, bool depth_model) {
  if (!stats_on(c, B)) return;
  const Plan& p = c->plan;
  a.stat_out = c->at<float>(depth_model ? p.dstat : p.hstat);
  a.stat_out_ld = depth_model ? p.dstat_ld : p.hstat_ld;
}

void enqueue_step(moshi_ctx* c, int B, bool depth) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  hipStream_t s = c->stream;
  const bool bf = p.bf;
  const int hdt = g.d_t / g.n_heads_t, hdd = g.d_d / g.n_heads_d;

  EmbedArgs ea{};
  ea.table = c->ws + p.emb_t;
  ea.row0 = c->at<long long>(p.meta_row0);
  ea.rows = c->at<int>(p.meta_rows);
  ea.frames = c->at<int>(p.st_prev);
  ea.h = c->at<float>(p.h);
  ea.d = g.d_t;
  ea.err = c->at<int>(p.st_err);
  if (stats_on(c, B)) {
    ea.stat_out = c->at<float>(p.hstat);
    ea.stat_ld = p.hstat_ld;
  }
  launch_embed(ea, B, bf, s);
  const int nh = p.hstat_ld, nd = p.dstat_ld;  // partials of a residual GEMV producer

  for (int l = 0; l < g.n_layers_t; ++l) {
    const LayerW& w = p.lt[l];
    GemvArgs qa = qkv_args(c, w, l, false, 0);  // RMSNorm, Wqkv, RoPE, KV append
    stat_consume(c, qa, B, false, l == 0 ? (g.d_t + 255) / 256 : nh);
    launch_gemv(qa, B, EPI_QKV, bf, s);
    // keys 0..pos, then h += Wo attn (at B = 1 the split merge runs in Wo's prologue)
    const AttnArgs at = attn_args(c, l, false, 0);
    GemvArgs wa = wo_args(c, w, false);
    stat_produce(c, wa, B, false);
    if (!launch_attn_wo(at, B, g.n_heads_t, hdt, bf, wa, bf, s)) {
      launch_attn_decode(at, B, g.n_heads_t, hdt, bf, s);
      launch_gemv(wa, B, EPI_RESID, bf, s);
    }
    GemvArgs ga = gu_args(c, w, false);  // SiLU(Wg n) * Wu n
    stat_consume(c, ga, B, false, nh);
    launch_gemv(ga, B, EPI_SWIGLU, bf, s);
    GemvArgs da = down_args(c, w, false);  // h += Wdown inter
    stat_produce(c, da, B, false);
    launch_gemv(da, B, EPI_RESID, bf, s);
  }
  // text head on z = RMSNorm(h), greedy text token
  GemvArgs ta = text_head_args(c);
  stat_consume(c, ta, B, false, nh);
  launch_gemv(ta, B, EPI_STORE, bf, s);
  launch_argmax(argmax_args(c, 0), B, s);
  if (depth) {
    for (int j = 0; j < depth_indices(g); ++j) {
      const DepthW& w = p.dj[j];
      // u_j = W_in^j z + E_D^j[token of slot j]
      GemvArgs a{};
      a.eps = g.norm_eps;
      set_weights(c, a, w.in_proj);
      a.N = g.d_d;
      a.K = g.d_t;
      a.x = c->at<float>(p.h);
      a.ldx = g.d_t;
      a.gain = c->at<float>(p.out_norm);
      a.y = c->at<float>(p.hd);
      a.ldy = g.d_d;
      a.emb = c->ws + w.emb;
      if (j < kSlots) {
        a.tok = c->at<int>(p.st_cur_tok);
        a.tok_stride = kSlots;
        a.tok_col = j;
      } else {  // the user's codebook j - 9 (given or drawn at index j - 1)
        a.tok = c->at<int>(p.st_user_cur);
        a.tok_stride = 8;
        a.tok_col = j - kSlots;
      }
      a.tok_rows = (j == 0 ? g.vocab_text : g.codebook) + 1;
      stat_consume(c, a, B, false, nh);
      stat_produce(c, a, B, true);
      launch_gemv(a, B, EPI_EMB, bf, s);
      for (int l = 0; l < g.n_layers_d; ++l) {
        const LayerW& lw = w.layers[l];
        GemvArgs dq = qkv_args(c, lw, l, true, j);
        stat_consume(c, dq, B, true, nd);
        launch_gemv(dq, B, EPI_QKV, bf, s);
        // attention over this frame's positions 0..j, then h += Wo attn (at
        // B = 1 the attention runs in Wo's prologue)
        const AttnArgs dat = attn_args(c, l, true, j);
        GemvArgs dwo = wo_args(c, lw, true);
        stat_produce(c, dwo, B, true);
        if (!launch_attn_wo(dat, B, g.n_heads_d, hdd, false, dwo, bf, s)) {
          launch_attn_decode(dat, B, g.n_heads_d, hdd, false, s);
          launch_gemv(dwo, B, EPI_RESID, bf, s);
        }
        GemvArgs dgu = gu_args(c, lw, true);
        stat_consume(c, dgu, B, true, nd);
        launch_gemv(dgu, B, EPI_SWIGLU, bf, s);
        GemvArgs ddn = down_args(c, lw, true);
        stat_produce(c, ddn, B, true);
        launch_gemv(ddn, B, EPI_RESID, bf, s);
      }
      GemvArgs hh{};
      hh.eps = g.norm_eps;
      set_weights(c, hh, w.head);
      hh.N = g.codebook;
      hh.K = g.d_d;
      hh.x = c->at<float>(p.hd);
      hh.ldx = g.d_d;
      hh.gain = c->at<float>(w.out_norm);
      hh.y = c->at<float>(p.audio_logits) + (long long)j * g.codebook;
      hh.ldy = depth_indices(g) * g.codebook;
      stat_consume(c, hh, B, true, nd);
      launch_gemv(hh, B, EPI_STORE, bf, s);
      launch_argmax(argmax_args(c, j + 1), B, s);
    }
  }
  AdvanceArgs av{};
  av.cur_tok = c->at<int>(p.st_cur_tok);
  av.force = c->at<int>(p.st_force);
  av.has_force = c->at<int>(p.st_has_force);
  av.user = c->at<int>(p.st_user);
  av.prev = c->at<int>(p.st_prev);
  av.pos = c->at<int>(p.st_pos);
  av.err = c->at<int>(p.st_err);
  av.pad_text = g.vocab_text;
  av.pad_audio = g.codebook;
  av.text_only = depth ? 0 : 1;
  av.out_tok = c->at<int>(p.st_out_tok);
  av.user_cur = depth && depth_indices(g) == 16 ? c->at<int>(p.st_user_cur) : nullptr;
  launch_advance(av, B, s);
  HIPCHECK(hipGetLastError());
}

// operands of one teacher-forced GEMM over M frames: the fp16 copy of weight W
GemmArgs tf_gemm_args(moshi_ctx* c, const void* W, const uint16_t* X, long long ldx, long long M, int N, int K) {
  GemmArgs a{};
  a.W = c->at<uint16_t>(c->plan.w16 + (size_t)((const char*)W - c->ws));
  a.X = X;
  a.ldx = ldx;
  a.M = (int)M;
  a.N = N;
  a.K = K;
  return a;
}

// causal flash attention of temporal layer l over S frames of each conversation
FlashArgs tf_flash_args(moshi_ctx* c, int l, int S) {
  const int d = c->cfg.d_t;
  FlashArgs fa{};
  fa.q = c->at<uint16_t>(c->plan.tf_Q);
  fa.ldq = d;
  fa.kv = temporal_kv(c);
  fa.layer = l;
  fa.S = S;
  fa.scale = 1.0f / sqrtf((float)(d / c->cfg.n_heads_t));
  fa.out = c->at<uint16_t>(c->plan.tf_O);
  fa.ldo = d;
  return fa;
}

// Teacher-forced pass on matrix cores (bf16 models): every linear map is one
// GEMM over the B*S frames; attention is causal flash attention over the KV
// pages of conversations 0..B-1; the Depth Transformer runs layer by layer over
// its 8 positions, which teacher forcing makes known in advance.
void enqueue_tf_mfma(moshi_ctx* c, const int* tok, int B, int S, bool depth, float* text_out, float* audio_out,
                     bool want_loss) {
  const moshi_config& g = c->cfg;
  const Plan& p = c->plan;
  hipStream_t s = c->stream;
  const long long M = (long long)B * S;
  const int d = g.d_t, F = g.ffn_t, dd = g.d_d, Fd = g.ffn_d, NQ = g.n_q;
  const int hdt = d / g.n_heads_t, hdd = dd / g.n_heads_d;
  float* H = c->at<float>(p.tf_H);
  uint16_t* Xn = c->at<uint16_t>(p.tf_Xn);
  uint16_t* I = c->at<uint16_t>(p.tf_I);
  uint16_t* Q = c->at<uint16_t>(p.tf_Q);
  uint16_t* O = c->at<uint16_t>(p.tf_O);
  float* text = text_out ? text_out : c->at<float>(p.tf_text);
  float* audio = audio_out ? audio_out : c->at<float>(p.tf_audio);

  EmbedArgs ea{};
  ea.table = c->ws + p.emb_t;
  ea.row0 = c->at<long long>(p.meta_row0);
  ea.rows = c->at<int>(p.meta_rows);
  ea.h = H;
  ea.d = d;
  ea.err = c->at<int>(p.st_err);
  launch_tf_embed(ea, tok, M, S, g.vocab_text, g.codebook, s);

  const KvView tkv = temporal_kv(c);
  auto gemm = [&](const void* W, const uint16_t* X, long long ldx, int N, int K) {
    return tf_gemm_args(c, W, X, ldx, M, N, K);
  };
  for (int l = 0; l < g.n_layers_t; ++l) {
    const LayerW& w = p.lt[l];
    launch_rmsnorm_f16(H, d, c->at<float>(w.attn_norm), g.norm_eps, d, Xn, d, M, s);
    GemmArgs q = gemm(c->ws + w.wqkv, Xn, d, 3 * d, d);
    q.d = d;
    q.hd = hdt;
    q.S = S;
    q.pos_const = -1;
    q.rope = c->at<float>(p.rope_t);
    q.q = Q;
    q.ldq = d;
    q.kv = tkv;
    q.kv_paged = 1;
    q.layer = l;
    launch_gemm_bf16(q, TF_QKV, s);
    launch_flash_attn(tf_flash_args(c, l, S), B, g.n_heads_t, hdt, s);
    GemmArgs o = gemm(c->ws + w.wo, O, d, d, d);
    o.Yf = H;
    o.ldy = d;
    launch_gemm_bf16(o, TF_RESID, s);
    launch_rmsnorm_f16(H, d, c->at<float>(w.ffn_norm), g.norm_eps, d, Xn, d, M, s);
    GemmArgs gu = gemm(c->ws + w.wgu, Xn, d, 2 * F, d);
    gu.Yb = I;
    gu.ldy = F;
    launch_gemm_bf16(gu, TF_SWIGLU, s);
    GemmArgs dn = gemm(c->ws + w.wdown, I, F, d, F);
    dn.Yf = H;
    dn.ldy = d;
    launch_gemm_bf16(dn, TF_RESID, s);
  }
  // z = RMSNorm(h) (kept in Xn for the depth input projections), text logits
  launch_rmsnorm_f16(H, d, c->at<float>(p.out_norm), g.norm_eps, d, Xn, d, M, s);
  GemmArgs th = gemm(c->ws + p.text_head, Xn, d, g.vocab_text, d);
  th.Yf = text;
  th.ldy = g.vocab_text;
  launch_gemm_bf16(th, TF_STORE_F32, s);

  if (depth) {
    float* U = c->at<float>(p.tf_U);
    uint16_t* Xd = c->at<uint16_t>(p.tf_Xd);
    uint16_t* DQ = c->at<uint16_t>(p.tf_DQ);
    uint16_t* DK = c->at<uint16_t>(p.tf_DK);
    uint16_t* DV = c->at<uint16_t>(p.tf_DV);
    uint16_t* DO = c->at<uint16_t>(p.tf_DO);
    uint16_t* DI = c->at<uint16_t>(p.tf_DI);
    for (int j = 0; j < NQ; ++j) {
      const DepthW& w = p.dj[j];
      GemmArgs a = gemm(c->ws + w.in_proj, Xn, d, dd, d);
      a.Yf = U + (long long)j * M * dd;
      a.ldy = dd;
      a.tok = tok + j;  // depth position j reads the true token of slot j
      a.tok_stride = kStreams;
      a.tok_rows = (j == 0 ? g.vocab_text : g.codebook) + 1;
      a.emb = c->at<uint16_t>(w.emb);
      launch_gemm_bf16(a, TF_EMB, s);
    }
    for (int l = 0; l < g.n_layers_d; ++l) {
      for (int j = 0; j < NQ; ++j) {
        const LayerW& lw = p.dj[j].layers[l];
        float* Uj = U + (long long)j * M * dd;
        launch_rmsnorm_f16(Uj, dd, c->at<float>(lw.attn_norm), g.norm_eps, dd, Xd, dd, M, s);
        GemmArgs q = gemm(c->ws + lw.wqkv, Xd, dd, 3 * dd, dd);
        q.d = dd;
        q.hd = hdd;
        q.S = S;
        q.pos_const = j;
        q.rope = c->at<float>(p.rope_d);
        q.q = DQ + (long long)j * M * dd;
        q.ldq = dd;
        q.kv_paged = 0;
        q.dk = DK + (long long)j * M * dd;
        q.dv = DV + (long long)j * M * dd;
        launch_gemm_bf16(q, TF_QKV, s);
      }
      for (int j = 0; j < NQ; ++j) {
        const LayerW& lw = p.dj[j].layers[l];
        float* Uj = U + (long long)j * M * dd;
        DepthAttnArgs da{};
        da.q = DQ;
        da.k = DK;
        da.v = DV;
        da.out = DO;
        da.M = M;
        da.d = dd;
        da.H = g.n_heads_d;
        da.hd = hdd;
        da.j = j;
        da.scale = 1.0f / sqrtf((float)hdd);
        launch_depth_attn(da, s);
        GemmArgs o = gemm(c->ws + lw.wo, DO, dd, dd, dd);
        o.Yf = Uj;
        o.ldy = dd;
        launch_gemm_bf16(o, TF_RESID, s);
        launch_rmsnorm_f16(Uj, dd, c->at<float>(lw.ffn_norm), g.norm_eps, dd, Xd, dd, M, s);
        GemmArgs gu = gemm(c->ws + lw.wgu, Xd, dd, 2 * Fd, dd);
        gu.Yb = DI;
        gu.ldy = Fd;
        launch_gemm_bf16(gu, TF_SWIGLU, s);
        GemmArgs dn = gemm(c->ws + lw.wdown, DI, Fd, dd, Fd);
        dn.Yf = Uj;
        dn.ldy = dd;
        launch_gemm_bf16(dn, TF_RESID, s);
      }
    }
    for (int j = 0; j < NQ; ++j) {
      const DepthW& w = p.dj[j];
      launch_rmsnorm_f16(U + (long long)j * M * dd, dd, c->at<float>(w.out_norm), g.norm_eps, dd, Xd, dd, M, s);
      GemmArgs hh = gemm(c->ws + w.head, Xd, dd, g.codebook, dd);
      hh.Yf = audio + (long long)j * g.codebook;
      hh.ldy = (long long)NQ * g.codebook;
      launch_gemm_bf16(hh, TF_STORE_F32, s);
    }
  }
  if (want_loss) {
    TfCeArgs ca{};
    ca.text_logits = text;
    ca.audio_logits = audio;
    ca.tokens = tok;
    ca.ce = c->at<double>(p.tf_ce);
    ca.vocab_text = g.vocab_text;
    ca.codebook = g.codebook;
    launch_tf_ce(ca, M, depth, s);
  }
  HIPCHECK(hipGetLastError());
}

void run_step(moshi_ctx* c, int B, bool depth) {
  if (!c->use_graph) {
    enqueue_step(c, B, depth);
    return;
  }
  auto key = std::make_pair(B, depth ? 1 : 0);
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    hipGraph_t graph;
    HIPCHECK(hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal));
    try {
      enqueue_step(c, B, depth);
    } catch (...) {
      (void)hipStreamEndCapture(c->stream, &graph);
      throw;
    }
    HIPCHECK(hipStreamEndCapture(c->stream, &graph));
    hipGraphExec_t exec;
    HIPCHECK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    HIPCHECK(hipGraphDestroy(graph));
    it = c->graphs.emplace(key, exec).first;
  }
  HIPCHECK(hipGraphLaunch(it->second, c->stream));
}

// make sure conversation b has KV pages for positions < upto
void ensure_pages(moshi_ctx* c, int b, int upto) {
  const int pf = c->cfg.page_frames;
  const int need = (upto + pf - 1) / pf;
  auto& pg = c->pages[b];
  while ((int)pg.size() < need) {
    if (c->free_pages.empty()) fail(MOSHI_ENOMEM, "KV page pool exhausted (%d pages)", c->plan.n_pages);
    const int phys = c->free_pages.back();
    c->free_pages.pop_back();
    const int idx = b * c->plan.max_pages_conv + (int)pg.size();
    pg.push_back(phys);
    c->pin_pt[idx] = phys;
    HIPCHECK(hipMemcpyAsync(c->at<int>(c->plan.page_table) + idx, c->pin_pt + idx, 4, hipMemcpyHostToDevice,
                            c->stream));
  }
}

void reset_conv(moshi_ctx* c, int b) {
  HIPCHECK(hipStreamSynchronize(c->stream));
  for (int ph : c->pages[b]) c->free_pages.push_back(ph);
  c->pages[b].clear();
  c->pos_h[b] = 0;
  if (c->cfg.tts_max_tokens) {
    int off[kTtsCtl] = {};
    HIPCHECK(hipMemcpy(c->at<int>(c->plan.tts_ctl) + b * kTtsCtl, off, sizeof off, hipMemcpyHostToDevice));
  }
  int frame[kStreams];
  frame[0] = c->cfg.vocab_text;
  for (int k = 1; k < kStreams; ++k) frame[k] = c->cfg.codebook;
  int zero = 0;
  HIPCHECK(hipMemcpy(c->at<int>(c->plan.st_prev) + b * kStreams, frame, sizeof frame, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(c->at<int>(c->plan.st_pos) + b, &zero, 4, hipMemcpyHostToDevice));
}

void check_ids(const int32_t* v, long long n, int stride, int first_slot, const moshi_config& g, int lo = 0) {
  for (long long i = 0; i < n; ++i) {
    const int slot = first_slot + (int)(i % stride);
    const int hi = slot == 0 ? g.vocab_text : g.codebook;
    if (v[i] < lo || v[i] > hi)
      fail(MOSHI_EINVAL, "token id %d out of range [%d, %d] in slot %d", v[i], lo, hi, slot);
  }
}

int guard_impl(moshi_ctx* c, const std::function<void()>& fn) {
  try {
    fn();
    return MOSHI_OK;
  } catch (const Error& e) {
    if (c) c->err = e.msg;
    return e.code;
  } catch (const std::exception& e) {
    if (c) c->err = e.what();
    return MOSHI_EINVAL;
  }
}
}  // namespace

extern "C" {

size_t moshi_workspace_bytes(const moshi_config* cfg) {
  if (!cfg) return 0;
  std::string msg;
  if (validate(*cfg, msg) != MOSHI_OK) return 0;
  return make_plan(*cfg).total;
}

int moshi_check_config(const moshi_config* cfg, char* msg, size_t msg_len) {
  std::string m;
  int rc = cfg ? validate(*cfg, m) : (m = "null config", MOSHI_EINVAL);
  if (msg && msg_len) {
    snprintf(msg, msg_len, "%s", m.c_str());
  }
  return rc;
}

int moshi_create(const moshi_config* cfg, void* hip_stream, void* workspace, size_t ws_bytes, moshi_ctx** out) {
  if (!out) {
    g_create_error = "out is null";
    return MOSHI_EINVAL;
  }
  *out = nullptr;
  if (!cfg) {
    g_create_error = "null config";
    return MOSHI_EINVAL;
  }
  std::string msg;
  if (validate(*cfg, msg) != MOSHI_OK) {
    g_create_error = msg;
    return MOSHI_EINVAL;
  }
  Plan plan = make_plan(*cfg);
  if (!workspace) {
    g_create_error = "workspace is null";
    return MOSHI_EINVAL;
  }
  if (ws_bytes < plan.total) {
    char buf[160];
    snprintf(buf, sizeof buf, "workspace of %zu bytes, %zu needed", ws_bytes, plan.total);
    g_create_error = buf;
    return MOSHI_ENOMEM;
  }
  moshi_ctx* c = new moshi_ctx();
  c->cfg = *cfg;
  c->plan = plan;
  c->ws = (char*)workspace;
  c->caller = (hipStream_t)hip_stream;
  const char* ng = getenv("MOSHI_NO_GRAPH");
  c->use_graph = !(ng && ng[0] == '1');
  const char* ts = getenv("MOSHI_TF_STEPS");
  c->tf_steps = ts && ts[0] == '1';
  int rc = guard_impl(c, [&] {
    HIPCHECK(hipGetDevice(&c->device));
    HIPCHECK(hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking));
    HIPCHECK(hipEventCreateWithFlags(&c->ev_in, hipEventDisableTiming));
    HIPCHECK(hipEventCreateWithFlags(&c->ev_out, hipEventDisableTiming));
    const Plan& p = c->plan;
    const int mb = cfg->max_batch;
    c->pinned_ints = mb * 8 + mb * kSlots + 1 + mb * kStreams + (size_t)mb * p.max_pages_conv + 2 + 64;
    HIPCHECK(hipHostMalloc((void**)&c->pinned, c->pinned_ints * 4 + 32 * 8, hipHostMallocDefault));
    c->pin_in = c->pinned;
    c->pin_out = c->pin_in + mb * 8 + mb * kSlots + 1;
    c->pin_pt = c->pin_out + mb * kStreams;
    c->pin_one = c->pin_pt + (size_t)mb * p.max_pages_conv;
    c->pin_zero = c->pin_one + 1;
    c->pin_res = (double*)(c->pinned + ((c->pinned_ints + 1) & ~(size_t)1));
    *c->pin_one = 1;
    *c->pin_zero = 0;
    build_dests(c);
    // state region: zero (attention counters must start at 0)
    HIPCHECK(hipMemsetAsync(c->ws + p.st_pos, 0, p.st_end - p.st_pos, c->stream));
    HIPCHECK(hipMemcpyAsync(c->ws + p.meta_row0, p.emb_row0, sizeof p.emb_row0, hipMemcpyHostToDevice, c->stream));
    HIPCHECK(hipMemcpyAsync(c->ws + p.meta_rows, p.emb_rows, sizeof p.emb_rows, hipMemcpyHostToDevice, c->stream));
    launch_rope_table(c->at<float>(p.rope_t), cfg->ctx_max, cfg->d_t / cfg->n_heads_t, cfg->rope_base, c->stream);
    launch_rope_table(c->at<float>(p.rope_d), depth_indices(*cfg), cfg->d_d / cfg->n_heads_d, cfg->rope_base,
                      c->stream);
    HIPCHECK(hipGetLastError());
    HIPCHECK(hipStreamSynchronize(c->stream));
    c->pos_h.assign(mb, 0);
    c->pages.assign(mb, {});
    for (int i = p.n_pages - 1; i >= 0; --i) c->free_pages.push_back(i);
    for (int b = 0; b < mb; ++b) reset_conv(c, b);
  });
  if (rc != MOSHI_OK) {
    g_create_error = c->err;
    moshi_destroy(c);
    return rc;
  }
  *out = c;
  return MOSHI_OK;
}

// 8-bit block format of a linear map (the walkthrough's "压缩Moshi及其对语音质量的
// 影响" section, "量化格式": asymmetric MinMax over blocks; block 32 and float16
// parameters per its Table 10 caption). Host code, float32 IEEE arithmetic:
// the weight is first rounded to bf16 (the model's precision), then per block
// scale = (max - min) / 255 and min are rounded to float16 and
// q = clamp(round_half_even((w - min16) / scale16), 0, 255); a flat block
// stores scale 0 and q = 0. Packs (scale | min << 16).
static uint16_t f32_to_f16_bits(float f) {
  const _Float16 h = (_Float16)f;
  uint16_t u;
  memcpy(&u, &h, 2);
  return u;
}
static float f16_bits_to_f32(uint16_t u) {
  _Float16 h;
  memcpy(&h, &u, 2);
  return (float)h;
}
static float bf16_round_host(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  float r;
  memcpy(&r, &u, 4);
  return r;
}
static void quantize_rows_q8(const float* src, long long rows, int cols, uint8_t* q, uint32_t* prm) {
  const int nb = cols / 32;
  auto work = [&](long long r_lo, long long r_hi) {
    float b[32];
    for (long long r = r_lo; r < r_hi; ++r) {
      for (int k = 0; k < nb; ++k) {
        const float* w = src + r * cols + k * 32;
        for (int i = 0; i < 32; ++i) b[i] = bf16_round_host(w[i]);
        float mn = b[0], mx = b[0];
        for (int i = 1; i < 32; ++i) {
          mn = std::min(mn, b[i]);
          mx = std::max(mx, b[i]);
        }
        const uint16_t s16 = f32_to_f16_bits((mx - mn) / 255.0f);
        const uint16_t m16 = f32_to_f16_bits(mn);
        const float sc = f16_bits_to_f32(s16), m = f16_bits_to_f32(m16);
        uint8_t* qo = q + r * cols + k * 32;
        for (int i = 0; i < 32; ++i) {
          float v = sc > 0.f ? nearbyintf((b[i] - m) / sc) : 0.f;
          v = std::min(255.f, std::max(0.f, v));
          qo[i] = (uint8_t)v;
        }
        prm[r * nb + k] = (uint32_t)s16 | ((uint32_t)m16 << 16);
      }
    }
  };
  const int nt = (int)std::max<long long>(1, std::min<long long>(16, rows / 64));
  std::vector<std::thread> th;
  for (int i = 0; i < nt; ++i) th.emplace_back(work, rows * i / nt, rows * (i + 1) / nt);
  for (auto& x : th) x.join();
}

// upload one linear map in 8-bit blocks (rows interleaved by mult/add as its
// dest says) and refresh its dequantised fp16 copy for the matrix-core pass
static void upload_q8(moshi_ctx* c, const Dest& ds, const moshi_tensor& t) {
  const Plan& p = c->plan;
  const long long rows = ds.rows, cols = ds.cols, nb = cols / 32;
  std::vector<float> host;
  const float* src = t.data;
  if (t.on_device) {
    host.resize((size_t)rows * cols);
    HIPCHECK(hipMemcpy(host.data(), t.data, host.size() * 4, hipMemcpyDeviceToHost));
    src = host.data();
  }
  std::vector<uint8_t> q((size_t)rows * cols);
  std::vector<uint32_t> prm((size_t)rows * nb);
  quantize_rows_q8(src, rows, (int)cols, q.data(), prm.data());
  // destination rows r * mult + add of the bf16 layout at ds.off
  char* qd = c->ws + p.q8w + ds.off / 2 + (size_t)ds.add * cols;
  char* pd = c->ws + p.q8p + ds.off / 16 + (size_t)ds.add * nb * 4;
  HIPCHECK(hipMemcpy2DAsync(qd, (size_t)ds.mult * cols, q.data(), cols, cols, rows, hipMemcpyHostToDevice, c->stream));
  HIPCHECK(hipMemcpy2DAsync(pd, (size_t)ds.mult * nb * 4, prm.data(), nb * 4, nb * 4, rows, hipMemcpyHostToDevice,
                            c->stream));
  if (p.tf_mfma)
    launch_q8_to_f16(c->at<uint8_t>(p.q8w + ds.off / 2), c->at<uint32_t>(p.q8p + ds.off / 16),
                     c->at<uint16_t>(p.w16 + ds.off), rows * ds.mult * cols, c->stream);
  HIPCHECK(hipGetLastError());
  HIPCHECK(hipStreamSynchronize(c->stream));  // the host buffers go out of scope
}

int moshi_init_weights(moshi_ctx* c, const moshi_tensor* t, int n) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    if (n < 0 || (n > 0 && !t)) fail(MOSHI_EINVAL, "bad tensor list");
    const Plan& p = c->plan;
    for (int i = 0; i < n; ++i) {
      if (!t[i].name || !t[i].data) fail(MOSHI_EINVAL, "tensor %d has no name or data", i);
      auto it = c->dests.find(t[i].name);
      if (it == c->dests.end()) fail(MOSHI_EINVAL, "unknown tensor name '%s'", t[i].name);
      Dest& ds = it->second;
      if (t[i].numel != ds.rows * ds.cols)
        fail(MOSHI_EINVAL, "tensor '%s' has %lld elements, %lld expected", t[i].name, (long long)t[i].numel,
             ds.rows * ds.cols);
      const bool bf = p.bf && !ds.f32;
      void* dst = c->ws + ds.off;
      if (p.q8 && ds.linear) {
        upload_q8(c, ds, t[i]);
      } else if (t[i].on_device) {
        launch_convert(t[i].data, ds.rows, ds.cols, dst, bf, ds.mult, ds.add, c->stream);
        HIPCHECK(hipGetLastError());
      } else {
        const long long chunk_rows = std::max<long long>(1, (long long)(p.staging_bytes / 4) / ds.cols);
        float* stg = c->at<float>(p.staging);
        for (long long r0 = 0; r0 < ds.rows; r0 += chunk_rows) {
          const long long nr = std::min(chunk_rows, ds.rows - r0);
          HIPCHECK(hipMemcpyAsync(stg, t[i].data + r0 * ds.cols, (size_t)nr * ds.cols * 4, hipMemcpyHostToDevice,
                                  c->stream));
          launch_convert(stg, nr, ds.cols, dst, bf, ds.mult, ds.add + r0 * ds.mult, c->stream);
          HIPCHECK(hipGetLastError());
          HIPCHECK(hipStreamSynchronize(c->stream));
        }
      }
      if (bf && p.tf_mfma && !(p.q8 && ds.linear)) {
        // the matrix-core pass reads an fp16 copy (same rounding as converting in the GEMM)
        launch_bf16_to_f16((const uint16_t*)dst, c->at<uint16_t>(p.w16 + ds.off), ds.rows * ds.mult * ds.cols,
                           c->stream);
        HIPCHECK(hipGetLastError());
      }
      if (!ds.loaded) {
        ds.loaded = true;
        ++c->n_loaded;
      }
    }
    HIPCHECK(hipStreamSynchronize(c->stream));
    c->ready = c->n_loaded == c->dests.size();
  });
}

int moshi_reset(moshi_ctx* c, int b) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    if (b < -1 || b >= c->cfg.max_batch) fail(MOSHI_EINVAL, "conversation %d out of range", b);
    if (b == -1)
      for (int i = 0; i < c->cfg.max_batch; ++i) reset_conv(c, i);
    else
      reset_conv(c, b);
  });
}

int moshi_step(moshi_ctx* c, int32_t B, const int32_t* user, const int32_t* force, int32_t* out_tokens,
               float* out_text, float* out_audio, int32_t flags) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    const moshi_config& g = c->cfg;
    const Plan& p = c->plan;
    if (!c->ready) fail(MOSHI_ESTATE, "weights not loaded");
    if (B < 1 || B > g.max_batch) fail(MOSHI_EINVAL, "batch %d out of range 1..%d", B, g.max_batch);
    const bool text_only = flags & MOSHI_STEP_TEXT_ONLY;
    const bool sim = depth_indices(g) == 16;  // the depth also draws the user's codebooks
    if (!out_tokens) fail(MOSHI_EINVAL, "out_tokens is required");
    if (!user && (!sim || text_only))
      fail(MOSHI_EINVAL, "user_codes are required unless a 16-index depth draws them");
    for (int b = 0; b < B; ++b)
      if (c->pos_h[b] + 1 > g.ctx_max) fail(MOSHI_ECONTEXT, "conversation %d is at ctx_max = %d", b, g.ctx_max);
    const bool dev = flags & MOSHI_DEVICE_PTRS;
    if (!dev) {
      if (user) check_ids(user, (long long)B * 8, 8, 9, g);
      if (force) check_ids(force, (long long)B * kSlots, kSlots, 0, g, -1);
    }
    if (text_only && out_audio) fail(MOSHI_EINVAL, "MOSHI_STEP_TEXT_ONLY computes no audio logits");
    order_in(c);
    for (int b = 0; b < B; ++b) ensure_pages(c, b, c->pos_h[b] + 1);
    hipStream_t s = c->stream;
    HIPCHECK(hipMemcpyAsync(c->ws + p.st_user_given, user ? c->pin_one : c->pin_zero, 4, hipMemcpyHostToDevice, s));
    if (dev) {
      if (user) HIPCHECK(hipMemcpyAsync(c->ws + p.st_user, user, (size_t)B * 8 * 4, hipMemcpyDeviceToDevice, s));
      if (force)
        HIPCHECK(hipMemcpyAsync(c->ws + p.st_force, force, (size_t)B * kSlots * 4, hipMemcpyDeviceToDevice, s));
      HIPCHECK(hipMemcpyAsync(c->ws + p.st_has_force, force ? c->pin_one : c->pin_zero, 4, hipMemcpyHostToDevice, s));
    } else {
      HIPCHECK(hipStreamSynchronize(s));  // the pinned input block may still be in use
      const int mb = g.max_batch;
      if (user) memcpy(c->pin_in, user, (size_t)B * 8 * 4);
      if (force) memcpy(c->pin_in + mb * 8, force, (size_t)B * kSlots * 4);
      c->pin_in[mb * 8 + mb * kSlots] = force ? 1 : 0;
      HIPCHECK(hipMemcpyAsync(c->ws + p.st_in, c->pin_in, (size_t)(mb * 8 + mb * kSlots + 1) * 4,
                              hipMemcpyHostToDevice, s));
    }
    run_step(c, B, !text_only);
    const hipMemcpyKind k = dev ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost;
    // own tokens: [B][9], or [B][17] with the user's draws (a text-only step
    // reports the given user codes there)
    const int row = sim ? kStreams : kSlots;
    int* otk = dev ? out_tokens : c->pin_out;
    HIPCHECK(hipMemcpy2DAsync(otk, (size_t)row * 4, c->ws + p.st_out_tok, kSlots * 4, kSlots * 4, B, k, s));
    if (sim)
      HIPCHECK(hipMemcpy2DAsync(otk + kSlots, (size_t)row * 4, c->ws + (text_only ? p.st_user : p.st_user_own), 8 * 4,
                                8 * 4, B, k, s));
    if (out_text) HIPCHECK(hipMemcpyAsync(out_text, c->ws + p.text_logits, (size_t)B * g.vocab_text * 4, k, s));
    if (out_audio)
      HIPCHECK(hipMemcpyAsync(out_audio, c->ws + p.audio_logits, (size_t)B * depth_indices(g) * g.codebook * 4, k,
                              s));
    for (int b = 0; b < B; ++b) c->pos_h[b] += 1;
    if (!dev) {
      HIPCHECK(hipStreamSynchronize(s));
      memcpy(out_tokens, c->pin_out, (size_t)B * row * 4);
    }
    order_out(c);
  });
}

int moshi_forward_teacher_forced(moshi_ctx* c, const int32_t* tokens, int32_t B, int32_t S, int32_t flags,
                                 float* text_logits, float* audio_logits, moshi_loss* loss) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    const moshi_config& g = c->cfg;
    const Plan& p = c->plan;
    if (!c->ready) fail(MOSHI_ESTATE, "weights not loaded");
    if (!tokens) fail(MOSHI_EINVAL, "tokens are required");
    if (B < 1 || B > g.max_batch) fail(MOSHI_EINVAL, "batch %d out of range 1..%d", B, g.max_batch);
    const long long tf_max = g.max_tf_tokens ? g.max_tf_tokens : (long long)g.ctx_max * g.max_batch;
    if (S < 1 || S > g.ctx_max) fail(MOSHI_EINVAL, "S = %d out of range 1..%d", S, g.ctx_max);
    if ((long long)B * S > tf_max) fail(MOSHI_EINVAL, "B*S = %lld exceeds max_tf_tokens %lld", (long long)B * S, tf_max);
    for (int b = 0; b < B; ++b)
      if (c->pos_h[b] != 0) fail(MOSHI_ESTATE, "conversation %d is not at position 0", b);
    const bool dev = flags & MOSHI_DEVICE_PTRS;
    const bool depth = !(flags & MOSHI_TF_SKIP_DEPTH);
    if (!dev) check_ids(tokens, (long long)B * S * kStreams, kStreams, 0, g);
    order_in(c);
    hipStream_t s = c->stream;
    const int* tok = tokens;
    if (!dev) {
      HIPCHECK(hipMemcpyAsync(c->ws + p.tf_tokens, tokens, (size_t)B * S * kStreams * 4, hipMemcpyHostToDevice, s));
      tok = c->at<int>(p.tf_tokens);
    }
    for (int b = 0; b < B; ++b) ensure_pages(c, b, S);
    const hipMemcpyKind k = dev ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost;
    if (p.tf_mfma && !c->tf_steps) {
      enqueue_tf_mfma(c, tok, B, S, depth, dev ? text_logits : nullptr, dev ? audio_logits : nullptr, loss != nullptr);
      c->tf_B = B;
      c->tf_S = S;
      if (!dev) {
        if (text_logits)
          HIPCHECK(hipMemcpyAsync(text_logits, c->ws + p.tf_text, (size_t)B * S * g.vocab_text * 4, k, s));
        if (audio_logits && depth)
          HIPCHECK(hipMemcpyAsync(audio_logits, c->ws + p.tf_audio, (size_t)B * S * g.n_q * g.codebook * 4, k, s));
      }
      if (flags & MOSHI_TF_FILL_KV) {
        // continue streaming at frame S+1: position S, previous frame V_S
        for (int b = 0; b < B; ++b) c->pin_in[b] = S;
        HIPCHECK(hipMemcpyAsync(c->ws + p.st_pos, c->pin_in, B * 4, hipMemcpyHostToDevice, s));
        HIPCHECK(hipMemcpy2DAsync(c->ws + p.st_prev, kStreams * 4, tok + (size_t)(S - 1) * kStreams,
                                  (size_t)S * kStreams * 4, kStreams * 4, B, hipMemcpyDeviceToDevice, s));
      }
    } else {
    HIPCHECK(hipMemcpyAsync(c->ws + p.st_has_force, c->pin_one, 4, hipMemcpyHostToDevice, s));
    HIPCHECK(hipMemcpyAsync(c->ws + p.st_user_given, c->pin_one, 4, hipMemcpyHostToDevice, s));
    for (int st = 0; st < S; ++st) {
      HIPCHECK(hipMemcpy2DAsync(c->ws + p.st_user, 8 * 4, tok + (size_t)st * kStreams + kSlots,
                                (size_t)S * kStreams * 4, 8 * 4, B, hipMemcpyDeviceToDevice, s));
      HIPCHECK(hipMemcpy2DAsync(c->ws + p.st_force, kSlots * 4, tok + (size_t)st * kStreams,
                                (size_t)S * kStreams * 4, kSlots * 4, B, hipMemcpyDeviceToDevice, s));
      run_step(c, B, depth);
      if (text_logits)
        HIPCHECK(hipMemcpy2DAsync(text_logits + (size_t)st * g.vocab_text, (size_t)S * g.vocab_text * 4,
                                  c->ws + p.text_logits, (size_t)g.vocab_text * 4, (size_t)g.vocab_text * 4, B, k, s));
      if (audio_logits && depth) {
        // Moshi's codebooks (a 16-index depth also wrote the user's after them)
        const size_t row = (size_t)g.n_q * g.codebook;
        HIPCHECK(hipMemcpy2DAsync(audio_logits + (size_t)st * row, (size_t)S * row * 4, c->ws + p.audio_logits,
                                  (size_t)depth_indices(g) * g.codebook * 4, row * 4, B, k, s));
      }
      if (loss) {
        CeRowsArgs ca{};
        ca.text_logits = c->at<float>(p.text_logits);
        ca.ld_text = g.vocab_text;
        ca.audio_logits = c->at<float>(p.audio_logits);
        ca.ld_audio = (long long)depth_indices(g) * g.codebook;
        ca.targets = c->at<int>(p.st_force);
        ca.tgt_stride = kSlots;
        ca.vocab_text = g.vocab_text;
        ca.codebook = g.codebook;
        ca.ce = c->at<double>(p.tf_ce);
        ca.S = S;
        ca.s = st;
        launch_ce_rows(ca, B, depth, s);
        HIPCHECK(hipGetLastError());
      }
    }
    }
    for (int b = 0; b < B; ++b) c->pos_h[b] = S;
    if (loss) {
      launch_ce_reduce(c->at<double>(p.tf_ce), (long long)B * S, depth ? kSlots : 1, c->at<double>(p.tf_res), s);
      HIPCHECK(hipGetLastError());
      HIPCHECK(hipMemcpyAsync(c->pin_res, c->ws + p.tf_res, 20 * 8, hipMemcpyDeviceToHost, s));
    }
    HIPCHECK(hipStreamSynchronize(s));
    if (loss) {
      const double* r = c->pin_res;
      loss->ce_text = r[0];
      for (int j = 0; j < 8; ++j) loss->ce_per_cb[j] = r[1 + j];
      loss->n_text = (int64_t)r[kSlots];
      long long na = 0;
      for (int j = 1; j < kSlots; ++j) na += (long long)r[kSlots + j];
      loss->n_audio = na;
      loss->ce_audio = r[18];
      loss->ce_total = r[19];
    }
    if (!(flags & MOSHI_TF_FILL_KV))
      for (int b = 0; b < B; ++b) reset_conv(c, b);
    order_out(c);
  });
}

int moshi_time_kernel(moshi_ctx* c, int32_t kernel, int32_t batch, int32_t iters, float* avg_us,
                      double* bytes_per_launch) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    const moshi_config& g = c->cfg;
    const Plan& p = c->plan;
    if (!c->ready) fail(MOSHI_ESTATE, "weights not loaded");
    if (batch < 1 || batch > g.max_batch) fail(MOSHI_EINVAL, "batch %d out of range", batch);
    if (iters < 1 || !avg_us || !bytes_per_launch) fail(MOSHI_EINVAL, "bad iters or output pointers");
    if (kernel < 0 || kernel > MOSHI_KERNEL_TF_ATTN) fail(MOSHI_EINVAL, "unknown kernel id %d", kernel);
    const bool tf = kernel >= MOSHI_KERNEL_TF_GATE_UP;
    if (tf && (!p.tf_mfma || c->tf_B == 0)) fail(MOSHI_ESTATE, "no matrix-core teacher-forced pass to time");
    if (tf && batch != c->tf_B) fail(MOSHI_EINVAL, "batch %d differs from the last teacher-forced pass (%d)", batch, c->tf_B);
    const double e = p.q8 ? 1.125 : p.esz;  // bytes per linear weight (8-bit codes + block parameters)
    const double d = g.d_t, F = g.ffn_t, B = batch;
    const long long tfM = (long long)c->tf_B * c->tf_S;
    const double S = c->tf_S;
    for (int b = 0; b < batch; ++b)
      if (kernel == MOSHI_KERNEL_ATTN && c->pos_h[b] < 1) fail(MOSHI_ESTATE, "attention timing needs a filled cache");
    double bytes = 0;
    auto enqueue = [&](int l) {
      const LayerW& w = p.lt[l];
      switch (kernel) {
        case MOSHI_KERNEL_QKV: {
          // time the projection only: the KV append writes into the page of the
          // next free position, which the next step overwrites anyway
          GemvArgs a = qkv_args(c, w, l, false, 0);
          stat_consume(c, a, batch, false, p.hstat_ld);
          launch_gemv(a, batch, EPI_QKV, p.bf, c->stream);
          bytes = 3 * d * d * e + B * (d * 4 + d * 4 + 2 * d * e);
          break;
        }
        case MOSHI_KERNEL_WO: {
          GemvArgs a = wo_args(c, w, false);
          stat_produce(c, a, batch, false);
          launch_gemv(a, batch, EPI_RESID, p.bf, c->stream);
          bytes = d * d * e + B * 3 * d * 4;
          break;
        }
        case MOSHI_KERNEL_FFN_GATE_UP: {
          GemvArgs a = gu_args(c, w, false);
          stat_consume(c, a, batch, false, p.hstat_ld);
          launch_gemv(a, batch, EPI_SWIGLU, p.bf, c->stream);
          bytes = 2 * F * d * e + B * (d + F) * 4;
          break;
        }
        case MOSHI_KERNEL_FFN_DOWN: {
          GemvArgs a = down_args(c, w, false);
          stat_produce(c, a, batch, false);
          launch_gemv(a, batch, EPI_RESID, p.bf, c->stream);
          bytes = d * F * e + B * (F + 2 * d) * 4;
          break;
        }
        case MOSHI_KERNEL_TEXT_HEAD: {
          GemvArgs a = text_head_args(c);
          stat_consume(c, a, batch, false, p.hstat_ld);
          launch_gemv(a, batch, EPI_STORE, p.bf, c->stream);
          bytes = g.vocab_text * d * e + B * (d + g.vocab_text) * 4;
          break;
        }
        case MOSHI_KERNEL_ATTN: {
          // keys 0..pos-1 of the filled cache: read K and V once
          launch_attn_decode(attn_args(c, l, false, 0), batch, g.n_heads_t, g.d_t / g.n_heads_t, p.bf, c->stream);
          double keys = 0;
          for (int b = 0; b < batch; ++b) keys += c->pos_h[b] + 1;
          bytes = keys * 2 * d * (p.bf ? 2 : 4) + B * 2 * d * 4;
          break;
        }
        case MOSHI_KERNEL_TF_GATE_UP: {
          GemmArgs gu = tf_gemm_args(c, c->ws + w.wgu, c->at<uint16_t>(p.tf_Xn), g.d_t, tfM, 2 * g.ffn_t, g.d_t);
          gu.Yb = c->at<uint16_t>(p.tf_I);
          gu.ldy = g.ffn_t;
          launch_gemm_bf16(gu, TF_SWIGLU, c->stream);
          bytes = 2.0 * (double)tfM * 2 * F * d;  // floating-point operations
          break;
        }
        case MOSHI_KERNEL_TF_ATTN:
          launch_flash_attn(tf_flash_args(c, l, c->tf_S), batch, g.n_heads_t, g.d_t / g.n_heads_t, c->stream);
          bytes = 4.0 * B * d * S * (S + 1) / 2;  // QK^T and PV over the causal pairs
          break;
      }
    };
    if (kernel == MOSHI_KERNEL_QKV)
      for (int b = 0; b < batch; ++b) ensure_pages(c, b, c->pos_h[b] + 1);  // the append stays in own pages
    hipEvent_t e0, e1;
    HIPCHECK(hipEventCreate(&e0));
    HIPCHECK(hipEventCreate(&e1));
    // the attention reads positions 0..pos[b]; pos is the next position, whose
    // key slot holds whatever the last step wrote there: stay inside the cache
    // by stepping the device position back by one for the timing
    if (kernel == MOSHI_KERNEL_ATTN) {
      for (int b = 0; b < batch; ++b) c->pin_in[b] = c->pos_h[b] - 1;
      HIPCHECK(hipMemcpyAsync(c->ws + p.st_pos, c->pin_in, batch * 4, hipMemcpyHostToDevice, c->stream));
    }
    for (int i = 0; i < g.n_layers_t; ++i) enqueue(i);  // warm
    HIPCHECK(hipEventRecord(e0, c->stream));
    for (int i = 0; i < iters; ++i) enqueue(i % g.n_layers_t);
    HIPCHECK(hipEventRecord(e1, c->stream));
    HIPCHECK(hipEventSynchronize(e1));
    float ms = 0;
    HIPCHECK(hipEventElapsedTime(&ms, e0, e1));
    if (kernel == MOSHI_KERNEL_ATTN) {
      for (int b = 0; b < batch; ++b) c->pin_in[b] = c->pos_h[b];
      HIPCHECK(hipMemcpyAsync(c->ws + p.st_pos, c->pin_in, batch * 4, hipMemcpyHostToDevice, c->stream));
      HIPCHECK(hipStreamSynchronize(c->stream));
    }
    HIPCHECK(hipEventDestroy(e0));
    HIPCHECK(hipEventDestroy(e1));
    HIPCHECK(hipGetLastError());
    *avg_us = ms * 1000.f / iters;
    *bytes_per_launch = bytes;
  });
}

int moshi_set_sampling(moshi_ctx* c, float temp_text, float temp_audio, uint64_t seed) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    if (!(temp_text >= 0.f) || !(temp_audio >= 0.f) || !std::isfinite(temp_text) || !std::isfinite(temp_audio))
      fail(MOSHI_EINVAL, "temperatures must be finite and >= 0");
    int32_t w[4];
    memcpy(&w[0], &temp_text, 4);
    memcpy(&w[1], &temp_audio, 4);
    w[2] = (int32_t)(uint32_t)(seed & 0xffffffffu);
    w[3] = (int32_t)(uint32_t)(seed >> 32);
    HIPCHECK(hipStreamSynchronize(c->stream));
    HIPCHECK(hipMemcpy(c->ws + c->plan.st_samp, w, sizeof w, hipMemcpyHostToDevice));
  });
}

int moshi_tts_text(moshi_ctx* c, int32_t conv, const int32_t* tokens, const int32_t* word_lens, int32_t n_words,
                   int32_t pad_id, int32_t epad_id, float target_pad_ratio, float bonus) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    const moshi_config& g = c->cfg;
    const Plan& p = c->plan;
    if (!g.tts_max_tokens) fail(MOSHI_EINVAL, "the context has no TTS text capacity (tts_max_tokens = 0)");
    if (conv < 0 || conv >= g.max_batch) fail(MOSHI_EINVAL, "conversation %d out of range", conv);
    if (n_words < 0 || (n_words > 0 && (!tokens || !word_lens))) fail(MOSHI_EINVAL, "bad word list");
    if (pad_id < 0 || pad_id >= g.vocab_text || epad_id < 0 || epad_id >= g.vocab_text)
      fail(MOSHI_EINVAL, "PAD and EPAD must be text ids in [0, %d)", g.vocab_text);
    if (!(bonus >= 0.f) || !std::isfinite(bonus) || !std::isfinite(target_pad_ratio))
      fail(MOSHI_EINVAL, "the bonus must be finite and >= 0, the target finite");
    long long n = 0;
    for (int w = 0; w < n_words; ++w) {
      if (word_lens[w] < 1) fail(MOSHI_EINVAL, "word %d is empty", w);
      n += word_lens[w];
    }
    if (n > g.tts_max_tokens) fail(MOSHI_EINVAL, "%lld text tokens exceed tts_max_tokens = %d", n, g.tts_max_tokens);
    std::vector<int32_t> start((size_t)n);
    for (long long i = 0, w = 0; w < n_words; ++w)
      for (int k = 0; k < word_lens[w]; ++k, ++i) {
        if (tokens[i] < 0 || tokens[i] >= g.vocab_text) fail(MOSHI_EINVAL, "text id %d out of range", tokens[i]);
        start[(size_t)i] = k == 0;
      }
    int32_t ctl[kTtsCtl] = {(int32_t)n, 0, 0, 0, pad_id, epad_id, 0, 0};
    memcpy(&ctl[6], &target_pad_ratio, 4);
    memcpy(&ctl[7], &bonus, 4);
    HIPCHECK(hipStreamSynchronize(c->stream));
    if (n) {
      HIPCHECK(hipMemcpy(c->at<int>(p.tts_tok) + (size_t)conv * g.tts_max_tokens, tokens, (size_t)n * 4,
                         hipMemcpyHostToDevice));
      HIPCHECK(hipMemcpy(c->at<int>(p.tts_start) + (size_t)conv * g.tts_max_tokens, start.data(), (size_t)n * 4,
                         hipMemcpyHostToDevice));
    }
    HIPCHECK(hipMemcpy(c->at<int>(p.tts_ctl) + conv * kTtsCtl, ctl, sizeof ctl, hipMemcpyHostToDevice));
  });
}

int moshi_read_q8(moshi_ctx* c, const char* name, uint8_t* codes, uint16_t* scale, uint16_t* mn) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    const Plan& p = c->plan;
    if (!p.q8) fail(MOSHI_EINVAL, "not an 8-bit model");
    if (!name || !codes || !scale || !mn) fail(MOSHI_EINVAL, "null argument");
    auto it = c->dests.find(name);
    if (it == c->dests.end() || !it->second.linear) fail(MOSHI_EINVAL, "'%s' is not a linear tensor", name);
    const Dest& ds = it->second;
    if (!ds.loaded) fail(MOSHI_EINVAL, "'%s' is not loaded", name);
    const long long rows = ds.rows, cols = ds.cols, nb = cols / 32;
    std::vector<uint32_t> prm((size_t)rows * nb);
    HIPCHECK(hipStreamSynchronize(c->stream));
    HIPCHECK(hipMemcpy2D(codes, cols, c->ws + p.q8w + ds.off / 2 + (size_t)ds.add * cols, (size_t)ds.mult * cols,
                         cols, rows, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy2D(prm.data(), nb * 4, c->ws + p.q8p + ds.off / 16 + (size_t)ds.add * nb * 4,
                         (size_t)ds.mult * nb * 4, nb * 4, rows, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < prm.size(); ++i) {
      scale[i] = (uint16_t)(prm[i] & 0xffffu);
      mn[i] = (uint16_t)(prm[i] >> 16);
    }
  });
}

int moshi_sync(moshi_ctx* c) {
  if (!c) return MOSHI_EINVAL;
  return guard_impl(c, [&] {
    HIPCHECK(hipStreamSynchronize(c->stream));
    int e = 0;
    HIPCHECK(hipMemcpy(&e, c->ws + c->plan.st_err, 4, hipMemcpyDeviceToHost));
    if (e) {
      int zero = 0;
      HIPCHECK(hipMemcpy(c->ws + c->plan.st_err, &zero, 4, hipMemcpyHostToDevice));
      fail(MOSHI_EINVAL, "a token id outside [0, pad] reached the device (replaced by pad)");
    }
  });
}

int moshi_position(const moshi_ctx* c, int b) {
  if (!c || b < 0 || b >= c->cfg.max_batch) return MOSHI_EINVAL;
  return c->pos_h[b];
}

int moshi_delay_codes(const int32_t* frames, int32_t T, int32_t tau, int32_t pad, int32_t* out) {
  if (T < 0 || tau < 0 || (T > 0 && (!frames || !out))) return MOSHI_EINVAL;
  for (int s = 0; s < T; ++s) {
    out[s * 8] = frames[s * 8];
    for (int q = 1; q < 8; ++q) out[s * 8 + q] = s - tau >= 0 ? frames[(s - tau) * 8 + q] : pad;
  }
  return MOSHI_OK;
}

int moshi_undelay_codes(const int32_t* model, int32_t T, int32_t tau, int32_t* out) {
  if (T < 0 || tau < 0 || (T > tau && (!model || !out))) return MOSHI_EINVAL;
  for (int t = 0; t + tau < T; ++t) {
    out[t * 8] = model[t * 8];
    for (int q = 1; q < 8; ++q) out[t * 8 + q] = model[(t + tau) * 8 + q];
  }
  return MOSHI_OK;
}

const char* moshi_last_error(const moshi_ctx* c) { return c ? c->err.c_str() : g_create_error.c_str(); }

void moshi_destroy(moshi_ctx* c) {
  if (!c) return;
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  if (c->pinned) (void)hipHostFree(c->pinned);
  if (c->ev_in) (void)hipEventDestroy(c->ev_in);
  if (c->ev_out) (void)hipEventDestroy(c->ev_out);
  if (c->stream) (void)hipStreamDestroy(c->stream);
  delete c;
}

}  // extern "C"
