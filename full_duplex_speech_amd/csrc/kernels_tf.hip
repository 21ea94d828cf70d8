// gfx950 kernels of the teacher-forced parallel pass (bf16 models).
//
// Teacher forcing ([W] "训练损失" of the Moshi paper walkthrough on 139.9.1.231:
// the model is trained on the joint sequence of eq. 6 given the true tokens)
// turns every linear map into a dense contraction over all B*S frames, so here
// the hot op is a matrix-core GEMM with the same fused epilogues as the
// streaming path (RoPE + KV append, SwiGLU, residual add), plus a causal
// flash-attention kernel on matrix cores.
//
// Operand precision: weights stay bf16 in HBM; the matrix cores take fp16
// operands (v_mfma_f32_32x32x16_f16, same rate as bf16 on gfx950) with fp32
// accumulation. Every bf16 weight value in fp16's normal range converts to
// fp16 exactly, and activations rounded to fp16 carry 3 more mantissa bits
// than bf16, which keeps a 32-layer pass within the parity tolerance. The
// residual stream, softmax statistics and logits stay fp32.
#include <hip/hip_runtime.h>

#include <math.h>

#include <stdexcept>

#include "moshi_internal.h"

namespace moshi {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t tf_f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float tf_bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ uint16_t tf_f2h(float f) {
  const _Float16 h = (_Float16)f;
  return *(const uint16_t*)&h;
}
__device__ __forceinline__ float tf_h2f(uint16_t v) { return (float)*(const _Float16*)&v; }
// 8 bf16 -> 8 fp16 (exact in fp16's normal range)
__device__ __forceinline__ u32x4t bf8_to_h8(u32x4t v) {
  u32x4t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    r[i] = (uint32_t)tf_f2h(__uint_as_float(w << 16)) | ((uint32_t)tf_f2h(__uint_as_float(w & 0xffff0000u)) << 16);
  }
  return r;
}

// ---------------------------------------------------------------------------
// C[m][n] = sum_k X[m][k] W[n][k]  (X fp16 [M][ldx], W fp16 [N][K], K % 64 == 0)
//
// The matrix core computes the transposed tile W_tile * X_tile^T: A operand =
// 32 rows of W, B operand = 32 rows of X, both read as 16-byte runs along K.
// In the result each lane holds, for one token m, four groups of four
// consecutive output features n -- so RoPE pairs and (gate, up) pairs sit in
// one lane and rows are written as 8- or 16-byte runs.
//
// Block: 256 threads = 4 waves in a 2 (n) x 2 (m) arrangement, each wave a
// (32 WT) x 64 tile (WT x 2 MFMA tiles), block tile (64 WT) (n) x 128 (m), K
// step kTK (64 where K allows), LDS double buffer filled from two register
// sets, so each step's loads are issued two steps before they are stored.
// WT = 2 measured best: the wider wave tile (WT = 4) needs 272+ registers and
// runs one wave per SIMD. Weights come from an fp16 copy made at upload, so
// both operands go to LDS without conversion. Blocks are ordered in groups of
// 8 tiles along m so that concurrently running blocks share both operand
// panels in L2.
// ---------------------------------------------------------------------------
constexpr int kTM = 128;

template <int EPI, int WT, int kTK, int PD>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmArgs g) {
  constexpr int kTN = 64 * WT;
  constexpr int kLdsRow = kTK + 8;        // padded row (fp16)
  constexpr int CPRW = kTK / 8;           // 16-byte chunks per row and K step
  constexpr int WCH = kTN * CPRW / 256;   // W chunks per thread and K step
  constexpr int XCH = kTM * CPRW / 256;   // X chunks per thread and K step
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kTN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kTM * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = g.M, N = g.N, K = g.K;
  // grouped rasterisation
  const int tiles_n = (N + kTN - 1) / kTN, tiles_m = (M + kTM - 1) / kTM;
  const int group = 16;  // measured: 8 -> 338 ms, 16 -> 328-330 ms, 24-32 -> 332-333 ms per 7B pass
  const int per_group = group * tiles_n;
  const int gid = blockIdx.x / per_group;
  const int first_m = gid * group;
  const int gsize = min(tiles_m - first_m, group);
  const int tm = first_m + (blockIdx.x % per_group) % gsize;
  const int tn = (blockIdx.x % per_group) / gsize;
  const int n0 = tn * kTN, m0 = tm * kTM;

  // global -> register loads: WCH chunks of 8 fp16 of W and 2 of X per thread
  // and K step, in two register sets: the loads of step kt + 2 are issued
  // while step kt is computed, so each has two steps of work to land. Steps
  // past the end re-read the last step (valid addresses, results unused), so
  // the loop carries no conditional loads.
  struct Regs {
    u32x4t w[WCH], x[XCH];
  };
  Regs ra, rb;
  const int nk = K / kTK;
  auto gload = [&](Regs& r, int kt) {
    const int k0 = min(kt, nk - 1) * kTK;
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CPRW, kc = (c % CPRW) * 8;
      r.w[i] = *(const u32x4t*)(g.W + (long long)min(n0 + row, N - 1) * K + k0 + kc);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CPRW, kc = (c % CPRW) * 8;
      r.x[i] = *(const u32x4t*)(g.X + (long long)min(m0 + row, M - 1) * g.ldx + k0 + kc);
    }
  };
  auto lstore = [&](const Regs& r, int buf) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4t*)(&Ws[buf][(c / CPRW) * kLdsRow + (c % CPRW) * 8]) = r.w[i];
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4t*)(&Xs[buf][(c / CPRW) * kLdsRow + (c % CPRW) * 8]) = r.x[i];
    }
  };

  const int wn = wave >> 1, wm = wave & 1;
  f32x16 acc[WT][2];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      f16x8 a[WT], b[2];
#pragma unroll
      for (int i = 0; i < WT; ++i) {
        const int row = wn * (32 * WT) + i * 32 + (lane & 31);
        a[i] = *(const f16x8*)(&Ws[buf][row * kLdsRow + ks * 16 + (lane >> 5) * 8]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wm * 64 + j * 32 + (lane & 31);
        b[j] = *(const f16x8*)(&Xs[buf][row * kLdsRow + ks * 16 + (lane >> 5) * 8]);
      }
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // nk is even (K % (2 kTK) == 0): the loop body is two steps and has no exits;
  // the last stores write re-read data that nothing reads
  if constexpr (PD == 1) {
    // one register set: the loads of step kt + 1 are issued before step kt is
    // computed (the last iteration re-reads the last step into an unused buffer)
    gload(ra, 0);
    lstore(ra, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      gload(ra, kt + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(kt & 1);
      lstore(ra, (kt & 1) ^ 1);
      __syncthreads();
    }
  } else {
  gload(ra, 0);
  gload(rb, 1);
  lstore(ra, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // step kt from LDS buffer 0; rb holds step kt + 1
    gload(ra, kt + 2);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the wait for rb
    compute(0);
    lstore(rb, 1);
    __syncthreads();
    // step kt + 1 from buffer 1; ra holds step kt + 2
    gload(rb, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    lstore(ra, 0);
    __syncthreads();
  }
  }

  // epilogue: lane holds token m = m0 + wm*64 + j*32 + lane%32 and features
  // n = n0 + wn*32*WT + i*32 + 8*q + 4*(lane/32) + t, for q, t in 0..3
#pragma unroll
  for (int i = 0; i < WT; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * 64 + j * 32 + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * (32 * WT) + i * 32 + 8 * q + 4 * (lane >> 5);
        if (n >= N) continue;
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if constexpr (EPI == TF_STORE_F32) {
          *(float4*)(g.Yf + (long long)m * g.ldy + n) = make_float4(v[0], v[1], v[2], v[3]);
        } else if constexpr (EPI == TF_RESID) {
          float4* p = (float4*)(g.Yf + (long long)m * g.ldy + n);
          float4 h = *p;
          h.x += v[0]; h.y += v[1]; h.z += v[2]; h.w += v[3];
          *p = h;
        } else if constexpr (EPI == TF_EMB) {
          const int t = min(max(g.tok[(long long)m * g.tok_stride], 0), g.tok_rows - 1);
          const uint16_t* e = g.emb + (long long)t * N + n;
          *(float4*)(g.Yf + (long long)m * g.ldy + n) =
              make_float4(v[0] + tf_bf2f(e[0]), v[1] + tf_bf2f(e[1]), v[2] + tf_bf2f(e[2]), v[3] + tf_bf2f(e[3]));
        } else if constexpr (EPI == TF_SWIGLU) {
          // (n, n+1) = (gate_i, up_i), i = n / 2
          const float a0 = v[0] / (1.0f + expf(-v[0])) * v[1];
          const float a1 = v[2] / (1.0f + expf(-v[2])) * v[3];
          *(uint32_t*)(g.Yb + (long long)m * g.ldy + (n >> 1)) = (uint32_t)tf_f2h(a0) | ((uint32_t)tf_f2h(a1) << 16);
        } else if constexpr (EPI == TF_QKV) {
          const int part = n / g.d;  // 0 q, 1 k, 2 v
          const int rr = n - part * g.d;
          const int head = rr / g.hd, dim = rr - head * g.hd;
          const int b = m / g.S, s = g.pos_const >= 0 ? g.pos_const : m - b * g.S;
          if (part < 2) {
#pragma unroll
            for (int p2 = 0; p2 < 2; ++p2) {
              const float* cs = g.rope + ((long long)s * (g.hd >> 1) + ((dim >> 1) + p2)) * 2;
              const float x0 = v[2 * p2], x1 = v[2 * p2 + 1];
              v[2 * p2] = x0 * cs[0] - x1 * cs[1];
              v[2 * p2 + 1] = x0 * cs[1] + x1 * cs[0];
            }
          }
          const bool to_cache = part > 0 && g.kv_paged;  // the KV cache is bf16
          const uint32_t lo = to_cache ? ((uint32_t)tf_f2bf(v[0]) | ((uint32_t)tf_f2bf(v[1]) << 16))
                                       : ((uint32_t)tf_f2h(v[0]) | ((uint32_t)tf_f2h(v[1]) << 16));
          const uint32_t hi = to_cache ? ((uint32_t)tf_f2bf(v[2]) | ((uint32_t)tf_f2bf(v[3]) << 16))
                                       : ((uint32_t)tf_f2h(v[2]) | ((uint32_t)tf_f2h(v[3]) << 16));
          uint16_t* dst;
          if (part == 0) {
            dst = g.q + (long long)m * g.ldq + rr;
          } else if (g.kv_paged) {
            const KvView& kv = g.kv;
            const int page = kv.page_table[b * kv.pt_stride + s / kv.pf];
            dst = (uint16_t*)kv.base + (long long)page * kv.page_stride +
                  ((long long)((g.layer * 2 + part - 1) * kv.n_heads + head) * kv.pf + (s % kv.pf)) * kv.hd + dim;
          } else {
            // flat [k|v][M][d] buffers (depth positions)
            dst = (part == 1 ? g.dk : g.dv) + (long long)m * g.d + rr;
          }
          *(uint2*)dst = make_uint2(lo, hi);
        }
      }
    }
  }
}

// fp16 copy of bf16 weights for the matrix-core pass
__global__ __launch_bounds__(256) void k_bf16_to_f16(const uint16_t* src, uint16_t* dst, long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    dst[i] = tf_f2h(tf_bf2f(src[i]));
}

void launch_bf16_to_f16(const uint16_t* src, uint16_t* dst, long long n, hipStream_t s) {
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  k_bf16_to_f16<<<(unsigned)blocks, 256, 0, s>>>(src, dst, n);
}

template <int WT, int KT, int PD>
static void gemm_launch(const GemmArgs& g, int epi, hipStream_t s) {
  const int tiles = ((g.N + 64 * WT - 1) / (64 * WT)) * ((g.M + kTM - 1) / kTM);
  switch (epi) {
    case TF_STORE_F32: k_gemm_bf16<TF_STORE_F32, WT, KT, PD><<<tiles, 256, 0, s>>>(g); break;
    case TF_RESID: k_gemm_bf16<TF_RESID, WT, KT, PD><<<tiles, 256, 0, s>>>(g); break;
    case TF_EMB: k_gemm_bf16<TF_EMB, WT, KT, PD><<<tiles, 256, 0, s>>>(g); break;
    case TF_SWIGLU: k_gemm_bf16<TF_SWIGLU, WT, KT, PD><<<tiles, 256, 0, s>>>(g); break;
    case TF_QKV: k_gemm_bf16<TF_QKV, WT, KT, PD><<<tiles, 256, 0, s>>>(g); break;
  }
}

void launch_gemm_bf16(const GemmArgs& g, int epi, hipStream_t s) {
  if (g.K % 64 != 0 || g.K <= 0) throw std::runtime_error("teacher-forced GEMM needs K % 64 == 0");
  // 64-wide K steps with two register sets need an even number of them
  if (g.K % 128 == 0)
    gemm_launch<2, 64, 2>(g, epi, s);
  else
    gemm_launch<2, 32, 2>(g, epi, s);
}

// ---------------------------------------------------------------------------
// Row-wise RMSNorm (float32 in) -> fp16 GEMM operand. One block per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm_f16(const float* x, long long ldx, const float* gain, float eps,
                                                      int D, uint16_t* y, long long ldy) {
  const long long r = blockIdx.x;
  const float* xr = x + r * ldx;
  __shared__ float red[4];
  float ss = 0.f;
  for (int k = threadIdx.x * 4; k < D; k += 1024) {
    const float4 v = *(const float4*)(xr + k);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)D + eps);
  for (int k = threadIdx.x * 4; k < D; k += 1024) {
    const float4 v = *(const float4*)(xr + k);
    const float4 gg = *(const float4*)(gain + k);
    const uint32_t lo = (uint32_t)tf_f2h(v.x * rs * gg.x) | ((uint32_t)tf_f2h(v.y * rs * gg.y) << 16);
    const uint32_t hi = (uint32_t)tf_f2h(v.z * rs * gg.z) | ((uint32_t)tf_f2h(v.w * rs * gg.w) << 16);
    *(uint2*)(y + r * ldy + k) = make_uint2(lo, hi);
  }
}

void launch_rmsnorm_f16(const float* x, long long ldx, const float* gain, float eps, int D, uint16_t* y,
                         long long ldy, long long rows, hipStream_t s) {
  k_rmsnorm_f16<<<(unsigned)rows, 256, 0, s>>>(x, ldx, gain, eps, D, y, ldy);
}

// ---------------------------------------------------------------------------
// Teacher-forced temporal inputs: row m = (b, s) sums the embeddings of
// V_{s-1} (s = 0: the all-pad initial frame). tokens [B][S][17].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_tf_embed(EmbedArgs a, const int* tokens, int S, int pad_text, int pad_audio) {
  const long long m = blockIdx.x;
  const int b = (int)(m / S), s = (int)(m - (long long)b * S);
  const int i = blockIdx.y * 256 + threadIdx.x;
  int t[kStreams];
#pragma unroll
  for (int k = 0; k < kStreams; ++k)
    t[k] = s == 0 ? (k == 0 ? pad_text : pad_audio) : tokens[((long long)b * S + s - 1) * kStreams + k];
  if (i >= a.d) return;
  float v[kStreams];
#pragma unroll
  for (int k = 0; k < kStreams; ++k) {
    const int tk = min(max(t[k], 0), a.rows[k] - 1);
    v[k] = tf_bf2f(((const uint16_t*)a.table)[(a.row0[k] + tk) * (long long)a.d + i]);
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kStreams; ++k) acc += v[k];
  a.h[m * a.d + i] = acc;
}

void launch_tf_embed(const EmbedArgs& a, const int* tokens, long long M, int S, int pad_text, int pad_audio,
                     hipStream_t s) {
  dim3 grid((unsigned)M, (a.d + 255) / 256);
  k_tf_embed<<<grid, 256, 0, s>>>(a, tokens, S, pad_text, pad_audio);
}

// ---------------------------------------------------------------------------
// Causal flash attention over the paged cache (bf16 K/V, fp16 Q and output).
// Block = QW waves = 32 QW queries of one (b, head); wave w owns queries
// q0 + 32w .. +31. Key tiles of 64 are staged in LDS (K as rows, V
// transposed); the next tile's K and V wait in registers while the current
// tile is computed. The matrix cores compute the transposed scores
// S^T = K Q^T, so each lane holds 32 scores of one query (the other 32 keys of
// the tile sit in lane l ^ 32) and the online-softmax statistics are in-lane
// reductions plus one exchange. The probabilities stay in registers as the B
// operand of O^T += V^T P^T: the contraction runs over the keys in the order
// the lanes hold them, and V^T is read from LDS in that order. Key tiles above
// a wave's diagonal are skipped; the longest query tiles are launched first.
// ---------------------------------------------------------------------------
constexpr int kFaKT = 64;
constexpr int kFaVRow = kFaKT + 4;  // V^T tile row (fp16): 34 words, conflict-free 8-byte reads

typedef uint32_t u32x2t __attribute__((ext_vector_type(2)));

// QW query waves per block (32 queries each): every staged K/V tile serves 32 QW queries
template <int HD, int QW>
__global__ __launch_bounds__(64 * QW, 8 / QW) void k_flash_attn(FlashArgs f) {
  constexpr int NT = 64 * QW;
  constexpr int kFaQT = 32 * QW;
  constexpr int KROW = HD + 8;                    // K tile row (fp16), padded
  constexpr int CPR = HD / 8;                     // 16-byte chunks per K/V row
  constexpr int KCH = kFaKT * CPR / NT;           // K chunks per thread and tile
  constexpr int VCH = (kFaKT / 2) * CPR / NT;     // V (key pair, chunk) units per thread and tile
  static_assert(KCH * NT == kFaKT * CPR && VCH * NT == (kFaKT / 2) * CPR, "staging must divide evenly");
  constexpr int TD = HD / 32;                     // 32-dim output blocks
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kFaKT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HD * kFaVRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5, ln = lane & 31;
  const int qt = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int S = f.S;
  const int q0 = qt * kFaQT, qw = q0 + wave * 32;
  const int myq = qw + ln;
  const KvView& kv = f.kv;
  const long long head_off = (long long)((f.layer * 2) * kv.n_heads + h) * kv.pf * kv.hd;
  const long long v_off = (long long)kv.n_heads * kv.pf * kv.hd;
  const uint16_t* kvb = (const uint16_t*)kv.base;
  // page ids of the keys 0..kend-1, so that tile fetches wait on nothing but themselves
  __shared__ int pages[kMaxPagesPerConv];
  const int kend = min(q0 + kFaQT, S);  // keys needed by this query tile
  for (int i = tid; i <= (kend - 1) / kv.pf; i += NT) pages[i] = kv.page_table[b * kv.pt_stride + i];
  __syncthreads();
  auto row_ptr = [&](int key) {
    return kvb + (long long)pages[key / kv.pf] * kv.page_stride + head_off + (long long)(key % kv.pf) * kv.hd;
  };

  // B operand of S^T = K Q^T: lane holds Q[myq][16 ks + 8 hl .. +7]
  f16x8 qf[HD / 16];
  {
    const uint16_t* qp = f.q + ((long long)b * S + min(myq, S - 1)) * f.ldq + h * HD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) qf[ks] = *(const f16x8*)(qp + 16 * ks);
  }

  u32x4t kreg[KCH], vreg[VCH][2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + NT * i;
      kreg[i] = *(const u32x4t*)(row_ptr(min(k0 + c / CPR, kend - 1)) + (c % CPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + NT * i, pr = c & 31, ch = c >> 5;
      vreg[i][0] = *(const u32x4t*)(row_ptr(min(k0 + 2 * pr, kend - 1)) + v_off + ch * 8);
      vreg[i][1] = *(const u32x4t*)(row_ptr(min(k0 + 2 * pr + 1, kend - 1)) + v_off + ch * 8);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + NT * i;
      *(u32x4t*)(&Ks[(c / CPR) * KROW + (c % CPR) * 8]) = bf8_to_h8(kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + NT * i, pr = c & 31, ch = c >> 5;
      const u32x4t v0 = bf8_to_h8(vreg[i][0]), v1 = bf8_to_h8(vreg[i][1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (v0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (v1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *(uint32_t*)(&Vt[(ch * 8 + e) * kFaVRow + 2 * pr]) = lo | (hi << 16);
      }
    }
  };

  f32x16 o[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float scale2 = f.scale * 1.4426950408889634f;  // log2(e)
  fetch(0);
  for (int k0 = 0; k0 < kend; k0 += kFaKT) {
    __syncthreads();  // the previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (k0 + kFaKT < kend) fetch(k0 + kFaKT);
    if (k0 > qw + 31) continue;  // whole tile above this wave's diagonal
    // S^T: sc[t][r] = S[myq][k0 + 32t + 8(r/4) + 4hl + r%4]
    f32x16 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const f16x8 kf = *(const f16x8*)(&Ks[(32 * t + ln) * KROW + 16 * ks + 8 * hl]);
        sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sc[t], 0, 0, 0);
      }
    }
    // scores in log2 units (scale * log2 e), so that exp(x) = 2^(x log2 e)
    // is one hardware exp2; only tiles that reach the diagonal or the end of
    // the sequence need the mask
    const bool masked = k0 + kFaKT - 1 > qw || k0 + kFaKT > S;
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = sc[t][r] * scale2;
        if (masked) {
          const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3);
          v = (key <= myq && key < S) ? v : -INFINITY;
        }
        sc[t][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // lazy rescaling: the reference maximum m moves only when a score exceeds
    // it by more than 2^8, so probabilities stay <= 256 and most tiles skip
    // rescaling the accumulators; l and o always share the same m
    const bool moved = mx > m + 8.f;  // m = -inf: any finite score moves it
    float alpha = 1.f;
    if (moved) {
      alpha = __builtin_amdgcn_exp2f(m - mx);  // 0 while nothing was accumulated
      m = mx;
    }
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[t][r] - m);
        sc[t][r] = pv;
        sum += pv;
      }
    sum += __shfl_xor(sum, 32, 64);
    l = l * alpha + sum;
    if (__any(moved)) {
#pragma unroll
      for (int t = 0; t < TD; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    }
    // O^T += V^T P^T over 4 steps of 16 keys; step ks holds the keys of
    // sc[ks / 2][8 (ks % 2) .. +7], i.e. k0 + 32 (ks/2) + 16 (ks%2) + 8 (i/4) + 4 hl + i%4
#pragma unroll
    for (int ks = 0; ks < kFaKT / 16; ++ks) {
      const int t = ks >> 1, rb = 8 * (ks & 1);
      f16x8 pf;
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[i] = (_Float16)sc[t][rb + i];
#pragma unroll
      for (int td = 0; td < TD; ++td) {
        const uint16_t* vp = &Vt[(32 * td + ln) * kFaVRow + 32 * t + 16 * (ks & 1) + 4 * hl];
        const u32x2t a0 = *(const u32x2t*)vp, a1 = *(const u32x2t*)(vp + 8);
        u32x4t av;
        av[0] = a0[0]; av[1] = a0[1]; av[2] = a1[0]; av[3] = a1[1];
        o[td] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)&av, pf, o[td], 0, 0, 0);
      }
    }
  }
  // O^T: o[td][r] = O[myq][32 td + 8 (r/4) + 4 hl + r%4]
  if (myq < S) {
    const float inv = 1.f / l;
    uint16_t* op = f.out + ((long long)b * S + myq) * f.ldo + h * HD + 4 * hl;
#pragma unroll
    for (int td = 0; td < TD; ++td)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2t w;
        w[0] = (uint32_t)tf_f2h(o[td][4 * g] * inv) | ((uint32_t)tf_f2h(o[td][4 * g + 1] * inv) << 16);
        w[1] = (uint32_t)tf_f2h(o[td][4 * g + 2] * inv) | ((uint32_t)tf_f2h(o[td][4 * g + 3] * inv) << 16);
        *(u32x2t*)(op + 32 * td + 8 * g) = w;
      }
  }
}

void launch_flash_attn(const FlashArgs& f, int B, int H, int hd, hipStream_t s) {
  // hd 128: 256 queries per block (943 -> 852 us per 7B layer against 128);
  // hd 64 stages too little per tile for 512 threads
  if (hd == 64)
    k_flash_attn<64, 4><<<dim3((f.S + 127) / 128, H, B), 256, 0, s>>>(f);
  else
    k_flash_attn<128, 8><<<dim3((f.S + 255) / 256, H, B), 512, 0, s>>>(f);
}

// ---------------------------------------------------------------------------
// Depth attention of the teacher-forced pass: frame m, depth position j, head
// h attends to positions 0..j of the same frame (at most 8). One wave per
// (m, head); q, k, v are bf16 [position][M][d] buffers.
// ---------------------------------------------------------------------------
// HD / 8 lanes per (m, head) item, 8 fp16 per lane; q, K and V of the j+1
// positions are requested together (positions past j re-read position j)
template <int HD>
__global__ __launch_bounds__(256) void k_depth_attn(DepthAttnArgs a) {
  constexpr int LPI = HD / 8, IPW = 64 / LPI;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane % LPI;
  const long long item = ((long long)blockIdx.x * 4 + wave) * IPW + lane / LPI;  // (m, head)
  const long long m = min(item / a.H, a.M - 1);
  const int h = (int)(item % a.H);
  const int j = a.j;
  const long long col = (long long)h * HD + li * 8;
  const u32x4t qr = *(const u32x4t*)(a.q + ((long long)j * a.M + m) * a.d + col);
  u32x4t kr[8], vr[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const long long off = ((long long)min(p, j) * a.M + m) * a.d + col;
    kr[p] = *(const u32x4t*)(a.k + off);
    vr[p] = *(const u32x4t*)(a.v + off);
  }
  float qf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] = tf_h2f((uint16_t)(qr[e >> 1] >> (16 * (e & 1))));
  float sc[8], mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf(qf[e], tf_h2f((uint16_t)(kr[p][e >> 1] >> (16 * (e & 1)))), d);
#pragma unroll
    for (int o = LPI / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
    sc[p] = d * a.scale;
    if (p <= j) mx = fmaxf(mx, sc[p]);
  }
  float l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (p <= j) {
      const float w = expf(sc[p] - mx);
      l += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(w, tf_h2f((uint16_t)(vr[p][e >> 1] >> (16 * (e & 1)))), o[e]);
    }
  }
  if (item >= (long long)a.M * a.H) return;
  const float inv = 1.f / l;
  u32x4t out;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    out[e] = (uint32_t)tf_f2h(o[2 * e] * inv) | ((uint32_t)tf_f2h(o[2 * e + 1] * inv) << 16);
  *(u32x4t*)(a.out + m * a.d + col) = out;
}

void launch_depth_attn(const DepthAttnArgs& a, hipStream_t s) {
  const long long items = (long long)a.M * a.H;
  if (a.hd == 64) {
    k_depth_attn<64><<<(unsigned)((items + 31) / 32), 256, 0, s>>>(a);
  } else if (a.hd == 32) {
    k_depth_attn<32><<<(unsigned)((items + 63) / 64), 256, 0, s>>>(a);
  } else if (a.hd == 16) {
    k_depth_attn<16><<<(unsigned)((items + 127) / 128), 256, 0, s>>>(a);
  } else {
    throw std::runtime_error("teacher-forced depth attention supports head dims 16, 32 and 64");
  }
}

// ---------------------------------------------------------------------------
// Cross-entropy rows of the teacher-forced pass: ce[m*9 + slot] =
// logsumexp(l) - l[target] or -1 for a pad target. Grid (M, 9).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_tf_ce(TfCeArgs a) {
  const long long m = blockIdx.x;
  const int slot = blockIdx.y, tid = threadIdx.x;
  const int n = slot == 0 ? a.vocab_text : a.codebook;
  const float* l = slot == 0 ? a.text_logits + m * a.vocab_text
                             : a.audio_logits + (m * 8 + (slot - 1)) * (long long)a.codebook;
  const int t = a.tokens[m * kStreams + slot];
  const int pad = n;
  double* out = a.ce + m * kSlots + slot;
  if (t < 0 || t >= pad) {
    if (tid == 0) *out = -1.0;
    return;
  }
  __shared__ float s_f[256];
  __shared__ double s_d[256];
  float mx = -INFINITY;
  for (int i = tid; i < n; i += 256) mx = fmaxf(mx, l[i]);
  s_f[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_f[tid] = fmaxf(s_f[tid], s_f[tid + o]);
    __syncthreads();
  }
  mx = s_f[0];
  double sum = 0.0;
  for (int i = tid; i < n; i += 256) sum += (double)expf(l[i] - mx);
  s_d[tid] = sum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_d[tid] += s_d[tid + o];
    __syncthreads();
  }
  if (tid == 0) *out = log(s_d[0]) + (double)mx - (double)l[t];
}

void launch_tf_ce(const TfCeArgs& a, long long M, bool with_audio, hipStream_t s) {
  dim3 grid((unsigned)M, with_audio ? kSlots : 1);
  k_tf_ce<<<grid, 256, 0, s>>>(a);
}

}  // namespace moshi
