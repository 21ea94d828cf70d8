// gfx950 kernels of the streaming frame step (batch 1..8).
//
// The step follows the RQ-Transformer of the Moshi paper walkthrough on
// 139.9.1.231 (section "使用 RQ-Transformer 的分层自回归建模", Fig. 3): a
// Helium-style Temporal Transformer ("Helium 文本语言模型 / 架构": RMSNorm at
// the attention, feed-forward and output-linear inputs, RoPE, causal attention,
// SiLU-gated linear unit) advances one position per frame, then a Depth
// Transformer with per-index weights produces Moshi's codebooks in order.
//
// At batch <= 8 every linear map is a weight-streaming matrix-vector product:
// HBM-bound, so the kernels are built around wide coalesced weight loads, not
// matrix cores.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>

#include <algorithm>

#include "moshi_internal.h"

namespace moshi {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
// float -> bfloat16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 16 bytes of weights -> EPL floats. Weights are read once per frame, so the
// loads are non-temporal.
template <bool BF>
struct WLoad;
template <>
struct WLoad<true> {
  static constexpr int EPL = 8;
  __device__ __forceinline__ static void get(const void* base, long long idx, float (&w)[8]) {
    u32x4 v = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)base + idx));
    w[0] = bf_lo(v.x); w[1] = bf_hi(v.x); w[2] = bf_lo(v.y); w[3] = bf_hi(v.y);
    w[4] = bf_lo(v.z); w[5] = bf_hi(v.z); w[6] = bf_lo(v.w); w[7] = bf_hi(v.w);
  }
};
template <>
struct WLoad<false> {
  static constexpr int EPL = 4;
  __device__ __forceinline__ static void get(const void* base, long long idx, float (&w)[4]) {
    f32x4 v = __builtin_nontemporal_load((const f32x4*)((const float*)base + idx));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
};

__device__ __forceinline__ float load_w1(const void* base, long long idx, bool bf) {
  return bf ? bf2f(((const uint16_t*)base)[idx]) : ((const float*)base)[idx];
}

// ---------------------------------------------------------------------------
// y = W * f(x) for NB input vectors; f = RMSNorm(.) * gain when gain != null.
// Block: 4 waves, each owning 4 consecutive output rows (so RoPE and SwiGLU
// pairs (2i, 2i+1) stay inside one wave). The normalised inputs are staged in
// LDS in K-chunks of KC elements; each lane streams 16-byte weight pieces and
// the wave reduces its rows with cross-lane shuffles.
// ---------------------------------------------------------------------------
constexpr int kGemvRowsPerWave = 4;
constexpr int kGemvRows = 4 * kGemvRowsPerWave;
constexpr int kGemvLdsFloats = 16384;

template <int NB, bool BF, int EPI, int RPW>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, int row0, int nrows, const float (&acc)[RPW][NB]) {
  const int N = a.N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float* y = a.y + (long long)b * a.ldy;
    if constexpr (EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_EMB) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int row = row0 + r;
        if (row >= N) break;
        float s = acc[r][b];
        if (EPI == EPI_RESID) s += y[row];
        if (EPI == EPI_EMB) {
          const int t = min(max(a.tok[b * a.tok_stride + a.tok_col], 0), a.tok_rows - 1);
          s += load_w1(a.emb, (long long)t * N + row, BF);
        }
        y[row] = s;
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      // rows (2i, 2i+1) = (gate_i, up_i)
#pragma unroll
      for (int r = 0; r < RPW; r += 2) {
        const int row = row0 + r;
        if (row + 1 >= N) break;
        const float g = acc[r][b], u = acc[r + 1][b];
        const float v = g / (1.0f + expf(-g)) * u;
        y[row >> 1] = v;
        if (a.y16) {
          const _Float16 hv = (_Float16)v;
          a.y16[(long long)b * a.ldy + (row >> 1)] = *(const uint16_t*)&hv;
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      const int p = a.pos ? a.pos[b] : a.pos_const;
#pragma unroll
      for (int r = 0; r < RPW; r += 2) {
        const int row = row0 + r;
        if (row + 1 >= N) break;
        float x0 = acc[r][b], x1 = acc[r + 1][b];
        const int part = row / a.d;  // 0 q, 1 k, 2 v
        const int rr = row - part * a.d;
        const int head = rr / a.hd, dim = rr - head * a.hd;
        if (part < 2) {
          const float* cs = a.rope + ((long long)p * (a.hd >> 1) + (dim >> 1)) * 2;
          const float c = cs[0], sn = cs[1];
          const float y0 = x0 * c - x1 * sn, y1 = x0 * sn + x1 * c;
          x0 = y0; x1 = y1;
        }
        if (part == 0) {
          y[rr] = x0;
          y[rr + 1] = x1;
        } else {
          const long long off = a.kv.offset(b, a.layer, part - 1, head, p) + dim;
          if (a.kv_bf16) {
            uint16_t* kv = (uint16_t*)a.kv.base;
            kv[off] = f2bf(x0);
            kv[off + 1] = f2bf(x1);
          } else {
            float* kv = (float*)a.kv.base;
            kv[off] = x0;
            kv[off + 1] = x1;
          }
        }
      }
    }
  }
}

template <int NB, bool BF, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a, int KC) {
  constexpr int EPL = WLoad<BF>::EPL;
  constexpr int RPW = kGemvRowsPerWave;
  extern __shared__ float xs[];  // [NB][kn]
  __shared__ float s_red[4][NB];
  __shared__ float s_rstd[NB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;

  if (a.gain) {
    float ss[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) ss[b] = 0.f;
    for (int k = tid; k < K; k += 256) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float v = a.x[(long long)b * a.ldx + k];
        ss[b] += v * v;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      ss[b] = wave_sum(ss[b]);
      if (lane == 0) s_red[wave][b] = ss[b];
    }
    __syncthreads();
    if (tid < NB) {
      float t = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
      s_rstd[tid] = 1.0f / sqrtf(t / (float)K + a.eps);
    }
    __syncthreads();
  }

  const int row0 = blockIdx.x * kGemvRows + wave * RPW;
  float acc[RPW][NB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    const int kn = min(KC, K - kc0);
    if (kc0) __syncthreads();
    for (int i = tid * 4; i < NB * kn; i += 1024) {
      const int b = i / kn, k = i - b * kn;
      float4 v = *(const float4*)(a.x + (long long)b * a.ldx + kc0 + k);
      if (a.gain) {
        const float r = s_rstd[b];
        const float4 g = *(const float4*)(a.gain + kc0 + k);
        v.x *= r * g.x; v.y *= r * g.y; v.z *= r * g.z; v.w *= r * g.w;
      }
      *(float4*)(xs + i) = v;
    }
    __syncthreads();
#pragma unroll 2
    for (int kk = lane * EPL; kk < kn; kk += 64 * EPL) {
      float w[RPW][EPL];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (row0 + r < N) {
          WLoad<BF>::get(a.W, (long long)(row0 + r) * K + kc0 + kk, w[r]);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) w[r][e] = 0.f;
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float xv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const float4 t = *(const float4*)(xs + b * kn + kk + e);
          xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[r][b] = fmaf(w[r][e], xv[e], acc[r][b]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
  if (lane != 0) return;

  gemv_epilogue<NB, BF, EPI, RPW>(a, row0, RPW, acc);
}

// Streaming variant used whenever the NB normalised input vectors fit in LDS
// (NB * K * 4 bytes <= 64 KB). Each wave owns one pair of output rows and walks
// K in groups of 8 wave-wide 16-byte loads per row; the loads of the next group
// are in flight while the current group is multiplied, and the first group is
// requested before the block's RMSNorm prologue so that HBM latency overlaps
// the prologue. One row pair per wave and many resident waves (8 per block)
// give the memory system the whole matrix's worth of requests at once.
constexpr int kStreamWaves = 8;

template <int NB, bool BF>
struct Unit {
  static constexpr int EPL = WLoad<BF>::EPL;
  static constexpr int SPAN = 64 * EPL;   // elements covered by one wave-wide load
  static constexpr int LPG = 8;           // loads per row per group
  static constexpr int GROUP = SPAN * LPG;
};

template <bool BF>
__device__ __forceinline__ void unpack16(const u32x4& v, float (&w)[WLoad<BF>::EPL]) {
  if constexpr (BF) {
    w[0] = bf_lo(v.x); w[1] = bf_hi(v.x); w[2] = bf_lo(v.y); w[3] = bf_hi(v.y);
    w[4] = bf_lo(v.z); w[5] = bf_hi(v.z); w[6] = bf_lo(v.w); w[7] = bf_hi(v.w);
  } else {
    w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y); w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
  }
}

template <int NB, bool BF, int EPI>
__global__ __launch_bounds__(64 * kStreamWaves) void k_gemv_stream(GemvArgs a) {
  using U = Unit<NB, BF>;
  constexpr int EPL = U::EPL, SPAN = U::SPAN, LPG = U::LPG, GROUP = U::GROUP;
  extern __shared__ float xs[];  // [NB][K]
  __shared__ float s_red[kStreamWaves][NB];
  __shared__ float s_rstd[NB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;
  const int row0 = (blockIdx.x * kStreamWaves + wave) * 2;
  const int ng = (K + GROUP - 1) / GROUP;
  const bool live = row0 < N;
  const bool has1 = row0 + 1 < N;
  const char* W0 = (const char*)a.W + (long long)row0 * K * (BF ? 2 : 4);
  const char* W1 = W0 + (long long)K * (BF ? 2 : 4);

  u32x4 wa[2][LPG], wb[2][LPG];
  auto load = [&](int g, u32x4 (&w)[2][LPG]) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int k = g * GROUP + i * SPAN + lane * EPL;
      const bool ok = k < K;
      const long long off = (long long)k * (BF ? 2 : 4);
      w[0][i] = (live && ok) ? __builtin_nontemporal_load((const u32x4*)(W0 + off)) : u32x4{0, 0, 0, 0};
      w[1][i] = (has1 && ok) ? __builtin_nontemporal_load((const u32x4*)(W1 + off)) : u32x4{0, 0, 0, 0};
    }
  };
  load(0, wa);

  // prologue: RMSNorm statistics and the normalised inputs in LDS
  float rs[NB];
  if (a.gain) {
#pragma unroll
    for (int b = 0; b < NB; ++b) rs[b] = 0.f;
    for (int k = tid * 4; k < K; k += 64 * kStreamWaves * 4) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 v = *(const float4*)(a.x + (long long)b * a.ldx + k);
        rs[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      rs[b] = wave_sum(rs[b]);
      if (lane == 0) s_red[wave][b] = rs[b];
    }
    __syncthreads();
    if (tid < NB) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kStreamWaves; ++w) t += s_red[w][tid];
      s_rstd[tid] = 1.0f / sqrtf(t / (float)K + a.eps);
    }
    __syncthreads();
  }
  for (int i = tid * 4; i < NB * K; i += 64 * kStreamWaves * 4) {
    const int b = i / K, k = i - b * K;
    float4 v = *(const float4*)(a.x + (long long)b * a.ldx + k);
    if (a.gain) {
      const float r = s_rstd[b];
      const float4 g = *(const float4*)(a.gain + k);
      v.x *= r * g.x; v.y *= r * g.y; v.z *= r * g.z; v.w *= r * g.w;
    }
    *(float4*)(xs + i) = v;
  }
  __syncthreads();
  if (!live) return;

  float acc[2][NB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

  auto consume = [&](int g, const u32x4 (&w)[2][LPG]) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int k = g * GROUP + i * SPAN + lane * EPL;
      if (k < K) {
        float w0[EPL], w1[EPL];
        unpack16<BF>(w[0][i], w0);
        unpack16<BF>(w[1][i], w1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float xv[EPL];
#pragma unroll
          for (int e = 0; e < EPL; e += 4) {
            const float4 t = *(const float4*)(xs + b * K + k + e);
            xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
          }
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            acc[0][b] = fmaf(w0[e], xv[e], acc[0][b]);
            acc[1][b] = fmaf(w1[e], xv[e], acc[1][b]);
          }
        }
      }
    }
  };
  for (int g = 0; g < ng; g += 2) {
    if (g + 1 < ng) load(g + 1, wb);
    consume(g, wa);
    if (g + 1 < ng) {
      if (g + 2 < ng) load(g + 2, wa);
      consume(g + 1, wb);
    }
  }

#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
  if (lane != 0) return;
  gemv_epilogue<NB, BF, EPI, 2>(a, row0, 2, acc);
}

// Outputs of one row pair (rows row, row + 1) of one input vector, given the
// two dot products s0, s1 and the pair's epilogue operands p0, p1 (residual,
// embedding row, or RoPE cos/sin).
template <int EPI>
__device__ __forceinline__ void pair_store(const GemvArgs& a, float* y, int row, float s0, float s1, float p0,
                                           float p1, int pos, int page) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_EMB) {
    y[row] = s0 + p0;
    if (row + 1 < a.N) y[row + 1] = s1 + p1;
  } else if constexpr (EPI == EPI_SWIGLU) {
    const float v = s0 / (1.0f + expf(-s0)) * s1;
    y[row >> 1] = v;
    if (a.y16) {
      const _Float16 hv = (_Float16)v;
      a.y16[(y - a.y) + (row >> 1)] = *(const uint16_t*)&hv;
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int part = row / a.d;
    const int rr = row - part * a.d;
    const int head = rr / a.hd, dim = rr - head * a.hd;
    float x0 = s0, x1 = s1;
    if (part < 2) {
      x0 = s0 * p0 - s1 * p1;
      x1 = s0 * p1 + s1 * p0;
    }
    if (part == 0) {
      y[rr] = x0;
      y[rr + 1] = x1;
    } else {
      const long long off = (long long)page * a.kv.page_stride +
                            ((long long)((a.layer * 2 + part - 1) * a.kv.n_heads + head) * a.kv.pf +
                             (pos % a.kv.pf)) * a.kv.hd + dim;
      if (a.kv_bf16) {
        const uint32_t v = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
        *(uint32_t*)((uint16_t*)a.kv.base + off) = v;
      } else {
        *(float2*)((float*)a.kv.base + off) = make_float2(x0, x1);
      }
    }
  }
}

// Where the prologue of a one-vector GEMV takes x from: XP_LOAD reads x (and
// applies the RMSNorm gain), XP_ATTN computes the depth attention itself,
// XP_MERGE merges the temporal attention's key-range partials.
constexpr int XP_LOAD = 0, XP_ATTN = 1, XP_MERGE = 2;
constexpr int kMergeMaxSplits = 8;

// Causal attention of NH heads h0, h0 + hs, ... of one query over the keys
// 0..P-1 (P <= NK) of a flat fp32 cache; lane = head dimension (hd <= 64),
// lanes past hd give 0; heads past H are not computed (their out is 0). q, K
// and V of all NH heads are requested together, so the wave waits on memory
// once; softmax with max subtraction.
template <int NK, int NH>
__device__ __forceinline__ void depth_attn_heads(const float* q, const KvView& kv, int b, int layer, int h0, int hs,
                                                 int H, int P, float scale, int lane, float (&out)[NH]) {
  const int hd = kv.hd;
  const bool on = lane < hd;
  const int dim = on ? lane : 0;
  const float* kvb = (const float*)kv.base;
  float qv[NH], kk[NH][NK], vv[NH][NK];
#pragma unroll
  for (int n = 0; n < NH; ++n) {
    const int h = min(h0 + n * hs, H - 1);
    const long long kb = kv.offset(b, layer, 0, h, 0) + dim;
    const long long vb = kv.offset(b, layer, 1, h, 0) + dim;
    qv[n] = q[h * hd + dim] * scale;
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      const int tt = min(t, P - 1);
      kk[n][t] = kvb[kb + (long long)tt * hd];
      vv[n][t] = kvb[vb + (long long)tt * hd];
    }
  }
#pragma unroll
  for (int n = 0; n < NH; ++n) {
    float sc[NK], m = -INFINITY;
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      sc[t] = wave_sum(on ? qv[n] * kk[n][t] : 0.f);
      if (t < P) m = fmaxf(m, sc[t]);
    }
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      if (t < P) {
        const float pr = expf(sc[t] - m);
        l += pr;
        o = fmaf(pr, vv[n][t], o);
      }
    }
    out[n] = on && h0 + n * hs < H ? o / l : 0.f;
  }
}

// x[k .. k+3] of the temporal attention output (k a multiple of 4, so the
// four values lie in one head): that head's key-range partials merged in split
// order, the arithmetic of the separate merge kernel; all partials are
// requested together
__device__ __forceinline__ float4 merge_x4(const GemvArgs& a, int k) {
  const int hd = a.hd, NS = a.merge_ns;
  const int h = k / hd, t = k - h * hd;
  const float* part = a.merge_part + (long long)h * NS * (hd + 2);
  float mx[kMergeMaxSplits], sm[kMergeMaxSplits], ov[kMergeMaxSplits][4];
#pragma unroll
  for (int i = 0; i < kMergeMaxSplits; ++i) {
    if (i < NS) {
      const float* pi = part + i * (hd + 2);
      mx[i] = pi[hd];
      sm[i] = pi[hd + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[i][e] = pi[t + e];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMergeMaxSplits; ++i)
    if (i < NS) M = fmaxf(M, mx[i]);
  float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMergeMaxSplits; ++i) {
    if (i < NS) {
      const float w = sm[i] > 0.f ? expf(mx[i] - M) : 0.f;
      L = fmaf(w, sm[i], L);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = fmaf(w, ov[i][e], o[e]);
    }
  }
  return make_float4(o[0] / L, o[1] / L, o[2] / L, o[3] / L);
}

// Persistent variant of the streaming GEMV: a grid of about two blocks per CU;
// every wave walks a sequence of units (row pair, K-group of LPG wave-wide
// loads per row) assigned round-robin over all waves. The weight registers of
// a unit are refilled with the next unit's data right after they are consumed,
// so each lane keeps ~2*LPG 16-byte loads in flight for the whole kernel. The
// steady-state loop has no data-dependent branches: addresses past the end of
// a row or of the matrix are clamped to valid weights whose products meet
// zero-padded inputs or are never stored, and every operand the epilogue
// needs (residual, embedding row, RoPE angle) is loaded before the refills,
// so the compiler never has to drain the load queue.
//
// KS = 2 (one input vector, a plain or residual store, at most one row pair per
// pair of waves): waves w and w + 4 of a block share a row pair and take its
// K-groups alternately, so maps with only 2048 row pairs (the 7B Wo and down
// projections) still keep 16 waves per CU streaming; the two partial sums
// meet in LDS and are added in wave order.
template <int NB, bool BF, int EPI, int LPG, int XP = XP_LOAD, int KS = 1>
__global__ __launch_bounds__(64 * kStreamWaves) void k_gemv_persist(GemvArgs a) {
  static_assert(XP == XP_LOAD || (XP == XP_MERGE && NB == 1), "the merge prologue takes one input vector");
  static_assert(KS == 1 || (KS == 2 && NB == 1 && (EPI == EPI_RESID || EPI == EPI_STORE)),
                "the split-K schedule takes one input vector and a plain or residual store");
  constexpr int G = kStreamWaves / KS;  // wave groups (row pairs in flight) per block
  __shared__ float s_ks[KS > 1 ? kStreamWaves : 1][2];
  constexpr int EPL = WLoad<BF>::EPL, SPAN = 64 * EPL, GROUP = SPAN * LPG;
  constexpr int ESZ = BF ? 2 : 4;
  extern __shared__ float4 xs4[];  // [NB][KP], zero past K
  float* xs = (float*)xs4;
  __shared__ float s_red[kStreamWaves][NB];
  __shared__ float s_rstd[NB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;
  const int ng = (K + GROUP - 1) / GROUP;
  const int KP = ng * GROUP;
  const int npairs = (N + 1) / 2;
  const int nw = gridDim.x * kStreamWaves;
  // row pairs go round-robin over the waves in wave-major order (wave w of
  // every block before wave w + 1 of any), so all blocks, and so all CUs, own
  // the same number of pairs to within one
  const int gw = wave * gridDim.x + blockIdx.x;
  // split-K schedule: wave group grp owns row pair gp, its wave ks the K-groups
  // ks, ks + KS, ...
  const int grp = wave % G, ks = wave / G;
  const int gp = grp * gridDim.x + blockIdx.x;
  const int mine = gw < npairs ? (npairs - 1 - gw) / nw + 1 : 0;
  const int units = KS > 1 ? (gp < npairs && ks < ng ? (ng - ks + KS - 1) / KS : 0) : mine * ng;
  const char* Wb = (const char*)a.W;

  // per-kernel epilogue constants
  int pos_b[NB], page_b[NB], tok_b[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    pos_b[b] = 0;
    page_b[b] = 0;
    tok_b[b] = 0;
    if constexpr (EPI == EPI_QKV) {
      pos_b[b] = a.pos ? a.pos[b] : a.pos_const;
      page_b[b] = a.kv.page_table ? a.kv.page_table[b * a.kv.pt_stride + pos_b[b] / a.kv.pf] : b;
    }
    if constexpr (EPI == EPI_EMB) tok_b[b] = min(max(a.tok[b * a.tok_stride + a.tok_col], 0), a.tok_rows - 1);
  }

  u32x4 w0[LPG], w1[LPG];
  auto load_slot = [&](int pair, int g, int i, u32x4& d0, u32x4& d1) {
    const int k = min(g * GROUP + i * SPAN + lane * EPL, K - EPL);
    const int r0 = min(pair * 2, N - 1), r1 = min(pair * 2 + 1, N - 1);
    d0 = __builtin_nontemporal_load((const u32x4*)(Wb + ((long long)r0 * K + k) * ESZ));
    d1 = __builtin_nontemporal_load((const u32x4*)(Wb + ((long long)r1 * K + k) * ESZ));
  };
  if (units > 0) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      if constexpr (KS > 1)
        load_slot(gp, ks, i, w0[i], w1[i]);
      else
        load_slot(gw, 0, i, w0[i], w1[i]);
    }
  }

  // prologue, one read of x: LDS gets gain * x (zero-padded) and the same pass
  // sums x^2; the RMSNorm factor 1/sqrt(mean(x^2) + eps) of conversation b is a
  // scalar of its outputs, applied to the dot products in the epilogue
  float rs[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) rs[b] = 0.f;
  for (int i = tid * 4; i < NB * KP; i += 64 * kStreamWaves * 4) {
    const int b = i / KP, k = i - b * KP;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (XP == XP_MERGE) {
      if (k < K) v = merge_x4(a, k);
    } else if (k < K) {
      v = *(const float4*)(a.x + (long long)b * a.ldx + k);
      if (a.gain) {
        const float q = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
          if (bb == b) rs[bb] += q;
        const float4 g = *(const float4*)(a.gain + k);
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      }
    }
    xs4[i >> 2] = v;
  }
  if (a.gain) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      rs[b] = wave_sum(rs[b]);
      if (lane == 0) s_red[wave][b] = rs[b];
    }
  }
  __syncthreads();
  if (a.gain && tid < NB) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) t += s_red[w][tid];
    s_rstd[tid] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
  if constexpr (KS > 1) {
    const float rs1 = a.gain ? s_rstd[0] : 1.f;
    const int r0 = min(gp * 2, N - 1), r1 = min(gp * 2 + 1, N - 1);
    float p0 = 0.f, p1 = 0.f;
    if (EPI == EPI_RESID && units > 0) {
      p0 = a.y[r0];
      p1 = a.y[r1];
    }
    float acc0 = 0.f, acc1 = 0.f;
    for (int u = 0; u < units; ++u) {
      const int g = ks + u * KS;
      const bool refill = u + 1 < units;
#pragma unroll
      for (int i = 0; i < LPG; ++i) {
        const int k = g * GROUP + i * SPAN + lane * EPL;
        float f0[EPL], f1[EPL], xv[EPL];
        unpack16<BF>(w0[i], f0);
        unpack16<BF>(w1[i], f1);
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const float4 t = xs4[(k + e) >> 2];
          xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          acc0 = fmaf(f0[e], xv[e], acc0);
          acc1 = fmaf(f1[e], xv[e], acc1);
        }
        if (refill) load_slot(gp, g + KS, i, w0[i], w1[i]);
      }
    }
    acc0 = wave_sum(acc0);
    acc1 = wave_sum(acc1);
    if (lane == 0) {
      s_ks[wave][0] = acc0;
      s_ks[wave][1] = acc1;
    }
    __syncthreads();
    if (ks != 0 || lane != 0 || gp >= npairs) return;
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      t0 += s_ks[q * G + grp][0];
      t1 += s_ks[q * G + grp][1];
    }
    pair_store<EPI>(a, a.y, gp * 2, t0 * rs1, t1 * rs1, p0, p1, 0, 0);
    return;
  }
  if (units == 0) return;
  float rstd[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) rstd[b] = a.gain ? s_rstd[b] : 1.f;

  float acc[2][NB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

  // epilogue operands of a row pair (residual, embedding row, RoPE angle); they
  // are loaded one row pair ahead and carried, so their loads are never
  // waited on right after the weight refills
  auto load_pre = [&](int pair, float (&pre)[2][NB]) {
    const int r0 = min(pair * 2, N - 1), r1 = min(pair * 2 + 1, N - 1);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      pre[0][b] = 0.f;
      pre[1][b] = 0.f;
      if constexpr (EPI == EPI_RESID) {
        pre[0][b] = a.y[(long long)b * a.ldy + r0];
        pre[1][b] = a.y[(long long)b * a.ldy + r1];
      }
      if constexpr (EPI == EPI_EMB) {
        pre[0][b] = load_w1(a.emb, (long long)tok_b[b] * N + r0, BF);
        pre[1][b] = load_w1(a.emb, (long long)tok_b[b] * N + r1, BF);
      }
      if constexpr (EPI == EPI_QKV) {
        // rows of q and k rotate; both rows of the pair share the angle
        const int dim = (r0 % a.d) % a.hd;
        const float* cs = a.rope + ((long long)pos_b[b] * (a.hd >> 1) + (dim >> 1)) * 2;
        pre[0][b] = cs[0];
        pre[1][b] = cs[1];
      }
    }
  };
  float pre[2][NB], pre_n[2][NB];
  load_pre(gw, pre);

  auto unit = [&](int pair, int g, int npair, int ngrp, bool refill) {
    if (refill) load_pre(npair, pre_n);
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int k = g * GROUP + i * SPAN + lane * EPL;
      float f0[EPL], f1[EPL];
      unpack16<BF>(w0[i], f0);
      unpack16<BF>(w1[i], f1);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float xv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const float4 t = xs4[(b * KP + k + e) >> 2];
          xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          acc[0][b] = fmaf(f0[e], xv[e], acc[0][b]);
          acc[1][b] = fmaf(f1[e], xv[e], acc[1][b]);
        }
      }
      if (refill) load_slot(npair, ngrp, i, w0[i], w1[i]);
    }
    if (g == ng - 1) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
      const int row = pair * 2;
      if (lane < NB) {
        // lane b stores conversation b's outputs
        const int b = lane;
        float s0 = acc[0][0], s1 = acc[1][0], p0 = pre[0][0], p1 = pre[1][0], r = rstd[0];
        int pos = pos_b[0], page = page_b[0];
#pragma unroll
        for (int bb = 1; bb < NB; ++bb)
          if (bb == b) {
            s0 = acc[0][bb]; s1 = acc[1][bb]; p0 = pre[0][bb]; p1 = pre[1][bb];
            pos = pos_b[bb]; page = page_b[bb]; r = rstd[bb];
          }
        pair_store<EPI>(a, a.y + (long long)b * a.ldy, row, s0 * r, s1 * r, p0, p1, pos, page);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
    }
    if (refill && ngrp == 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) pre[r][b] = pre_n[r][b];
    }
  };

  int pair = gw, g = 0;
  for (int u = 0; u < units - 1; ++u) {
    int npair = pair, ngrp = g + 1;
    if (ngrp == ng) {
      ngrp = 0;
      npair += nw;
    }
    unit(pair, g, npair, ngrp, true);
    pair = npair;
    g = ngrp;
  }
  unit(pair, g, pair, g, false);
}


// Split-K variant for one input vector and matrices with fewer row pairs than
// the chip has waves (the depth model's 1024-row maps, the depth heads): a
// block holds RG = 8/SK row pairs with SK waves each; wave s of a pair takes
// the K spans s, s+SK, s+2SK, ... (at most SPW of them, every lane one
// 16-byte load per row and span), so each block streams only a few KB and all
// CUs share the matrix. All weight loads are issued before the RMSNorm
// prologue; spans past K read clamped addresses against zero-padded inputs.
// The SK partial sums meet in LDS and are added in wave order.
template <bool BF, int EPI, int SPW, int XP = XP_LOAD>
__global__ __launch_bounds__(64 * kStreamWaves) void k_gemv_splitk(GemvArgs a, int SK) {
  constexpr int EPL = WLoad<BF>::EPL, SPAN = 64 * EPL, ESZ = BF ? 2 : 4;
  extern __shared__ float4 xs4[];  // [SK * SPW * SPAN], zero past K
  __shared__ float s_part[kStreamWaves][2];
  __shared__ float s_red[kStreamWaves];
  __shared__ float s_rstd;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;
  const int KPAD = SK * SPW * SPAN;
  const int RG = kStreamWaves / SK;
  const int npairs = (N + 1) / 2;
  const int pair = blockIdx.x * RG + wave / SK, sw = wave % SK;
  const int pr = min(pair, npairs - 1);
  const int r0 = min(pr * 2, N - 1), r1 = min(pr * 2 + 1, N - 1);
  const char* Wb = (const char*)a.W;

  u32x4 w0[SPW], w1[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = min((sw + i * SK) * SPAN + lane * EPL, K - EPL);
    w0[i] = __builtin_nontemporal_load((const u32x4*)(Wb + ((long long)r0 * K + k) * ESZ));
    w1[i] = __builtin_nontemporal_load((const u32x4*)(Wb + ((long long)r1 * K + k) * ESZ));
  }
  // epilogue operands of the pair
  float p0 = 0.f, p1 = 0.f;
  int pos = 0, page = 0;
  if constexpr (EPI == EPI_RESID) {
    p0 = a.y[r0];
    p1 = a.y[r1];
  }
  if constexpr (EPI == EPI_EMB) {
    const int t = min(max(a.tok[a.tok_col], 0), a.tok_rows - 1);
    p0 = load_w1(a.emb, (long long)t * N + r0, BF);
    p1 = load_w1(a.emb, (long long)t * N + r1, BF);
  }
  if constexpr (EPI == EPI_QKV) {
    pos = a.pos ? a.pos[0] : a.pos_const;
    page = a.kv.page_table ? a.kv.page_table[pos / a.kv.pf] : 0;
    const int dim = (r0 % a.d) % a.hd;
    const float* cs = a.rope + ((long long)pos * (a.hd >> 1) + (dim >> 1)) * 2;
    p0 = cs[0];
    p1 = cs[1];
  }

  // one read of x: LDS gets gain * x (zero-padded) and the same pass sums x^2;
  // the RMSNorm factor scales the dot products in the epilogue
  float rs = 0.f;
  if constexpr (XP == XP_ATTN) {
    // x = the depth attention output: wave w takes heads w, w + 8, ...
    for (int k = K + tid * 4; k < KPAD; k += 64 * kStreamWaves * 4) xs4[k >> 2] = make_float4(0.f, 0.f, 0.f, 0.f);
    // (two heads at a time, their loads in flight together)
    float* xs = (float*)xs4;
    const int P = a.pos_const + 1, H = K / a.hd;
    for (int h = wave; h < H; h += 2 * kStreamWaves) {
      float o[2];
      if (P <= 8)
        depth_attn_heads<8, 2>(a.attn_q, a.kv, 0, a.layer, h, kStreamWaves, H, P, a.attn_scale, lane, o);
      else
        depth_attn_heads<16, 2>(a.attn_q, a.kv, 0, a.layer, h, kStreamWaves, H, P, a.attn_scale, lane, o);
      if (lane < a.hd) {
        xs[h * a.hd + lane] = o[0];
        if (h + kStreamWaves < H) xs[(h + kStreamWaves) * a.hd + lane] = o[1];
      }
    }
  }
  for (int k = tid * 4; XP != XP_ATTN && k < KPAD; k += 64 * kStreamWaves * 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (XP == XP_MERGE && k < K) {
      v = merge_x4(a, k);
    } else if (k < K) {
      v = *(const float4*)(a.x + k);
      if (a.gain) {
        rs += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        const float4 g = *(const float4*)(a.gain + k);
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      }
    }
    xs4[k >> 2] = v;
  }
  if (a.gain) {
    rs = wave_sum(rs);
    if (lane == 0) s_red[wave] = rs;
  }
  __syncthreads();
  if (a.gain && tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) t += s_red[w];
    s_rstd = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
  const float rstd = a.gain ? s_rstd : 1.f;

  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = (sw + i * SK) * SPAN + lane * EPL;
    float f0[EPL], f1[EPL], xv[EPL];
    unpack16<BF>(w0[i], f0);
    unpack16<BF>(w1[i], f1);
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 t = xs4[(k + e) >> 2];
      xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc0 = fmaf(f0[e], xv[e], acc0);
      acc1 = fmaf(f1[e], xv[e], acc1);
    }
  }
  acc0 = wave_sum(acc0);
  acc1 = wave_sum(acc1);
  if (lane == 0) {
    s_part[wave][0] = acc0;
    s_part[wave][1] = acc1;
  }
  __syncthreads();
  if (sw != 0 || lane != 0 || pair >= npairs) return;
  float t0 = 0.f, t1 = 0.f;
  for (int w = 0; w < SK; ++w) {
    t0 += s_part[wave + w][0];
    t1 += s_part[wave + w][1];
  }
  pair_store<EPI>(a, a.y, pair * 2, t0 * rstd, t1 * rstd, p0, p1, pos, page);
}

// ---------------------------------------------------------------------------
// Weight-streaming GEMV over 8-bit block weights, one input vector (the
// 8-bit format of the walkthrough's "压缩Moshi及其对语音质量的影响" section:
// asymmetric MinMax over blocks of 32 weights of a row, scale and min in
// float16, w = q * scale + min). Each lane loads 16 codes (half a block) and
// that block's parameters, and adds scale * sum(q x) + min * sum(x) for its
// 16 inputs. Blocks hold RG = 8/SK row pairs with SK waves each; wave s of a
// pair takes the 1024-wide K spans s, s+SK, ... (at most SPW). The prologue
// and epilogues are the streaming kernels' (one read of x, RMSNorm factor on
// the dot products, pair_store).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_lo(uint32_t v) {
  const uint16_t h = (uint16_t)(v & 0xffffu);
  return (float)*(const _Float16*)&h;
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  const uint16_t h = (uint16_t)(v >> 16);
  return (float)*(const _Float16*)&h;
}

template <int EPI, int SPW>
__global__ __launch_bounds__(64 * kStreamWaves) void k_gemv_q8(GemvArgs a, int SK) {
  constexpr int EPL = 16, SPAN = 64 * EPL;
  extern __shared__ float4 xs4[];  // [SK * SPW * SPAN], zero past K
  __shared__ float s_part[kStreamWaves][2];
  __shared__ float s_red[kStreamWaves];
  __shared__ float s_rstd;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;
  const int KPAD = SK * SPW * SPAN;
  const int RG = kStreamWaves / SK;
  const int npairs = (N + 1) / 2;
  const int pair = blockIdx.x * RG + wave / SK, sw = wave % SK;
  const int pr = min(pair, npairs - 1);
  const int r0 = min(pr * 2, N - 1), r1 = min(pr * 2 + 1, N - 1);
  const uint8_t* Wq = (const uint8_t*)a.W;

  u32x4 w0[SPW], w1[SPW];
  uint32_t q0[SPW], q1[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = min((sw + i * SK) * SPAN + lane * EPL, K - EPL);
    w0[i] = __builtin_nontemporal_load((const u32x4*)(Wq + (long long)r0 * K + k));
    w1[i] = __builtin_nontemporal_load((const u32x4*)(Wq + (long long)r1 * K + k));
    q0[i] = a.Wq8p[((long long)r0 * K + k) >> 5];
    q1[i] = a.Wq8p[((long long)r1 * K + k) >> 5];
  }
  float p0 = 0.f, p1 = 0.f;
  int pos = 0, page = 0;
  if constexpr (EPI == EPI_RESID) {
    p0 = a.y[r0];
    p1 = a.y[r1];
  }
  if constexpr (EPI == EPI_EMB) {
    const int t = min(max(a.tok[a.tok_col], 0), a.tok_rows - 1);
    p0 = bf2f(((const uint16_t*)a.emb)[(long long)t * N + r0]);
    p1 = bf2f(((const uint16_t*)a.emb)[(long long)t * N + r1]);
  }
  if constexpr (EPI == EPI_QKV) {
    pos = a.pos ? a.pos[0] : a.pos_const;
    page = a.kv.page_table ? a.kv.page_table[pos / a.kv.pf] : 0;
    const int dim = (r0 % a.d) % a.hd;
    const float* cs = a.rope + ((long long)pos * (a.hd >> 1) + (dim >> 1)) * 2;
    p0 = cs[0];
    p1 = cs[1];
  }

  float rs = 0.f;
  for (int k = tid * 4; k < KPAD; k += 64 * kStreamWaves * 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < K) {
      v = *(const float4*)(a.x + k);
      if (a.gain) {
        rs += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        const float4 g = *(const float4*)(a.gain + k);
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      }
    }
    xs4[k >> 2] = v;
  }
  if (a.gain) {
    rs = wave_sum(rs);
    if (lane == 0) s_red[wave] = rs;
  }
  __syncthreads();
  if (a.gain && tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) t += s_red[w];
    s_rstd = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
  const float rstd = a.gain ? s_rstd : 1.f;

  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = (sw + i * SK) * SPAN + lane * EPL;
    float xv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 t = xs4[(k + e) >> 2];
      xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
    }
    float sx = 0.f, d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const uint32_t c0 = (w0[i][e >> 2] >> (8 * (e & 3))) & 0xffu;
      const uint32_t c1 = (w1[i][e >> 2] >> (8 * (e & 3))) & 0xffu;
      sx += xv[e];
      d0 = fmaf((float)c0, xv[e], d0);
      d1 = fmaf((float)c1, xv[e], d1);
    }
    acc0 = fmaf(f16_lo(q0[i]), d0, fmaf(f16_hi(q0[i]), sx, acc0));
    acc1 = fmaf(f16_lo(q1[i]), d1, fmaf(f16_hi(q1[i]), sx, acc1));
  }
  acc0 = wave_sum(acc0);
  acc1 = wave_sum(acc1);
  if (lane == 0) {
    s_part[wave][0] = acc0;
    s_part[wave][1] = acc1;
  }
  __syncthreads();
  if (sw != 0 || lane != 0 || pair >= npairs) return;
  float t0 = 0.f, t1 = 0.f;
  for (int w = 0; w < SK; ++w) {
    t0 += s_part[wave + w][0];
    t1 += s_part[wave + w][1];
  }
  pair_store<EPI>(a, a.y, pair * 2, t0 * rstd, t1 * rstd, p0, p1, pos, page);
}

// Persistent 8-bit variant for matrices with at least as many row pairs as the
// chip runs waves (the temporal maps, the text head): the streaming kernels'
// persistent schedule (units of one row pair and LPG 1024-wide spans, dealt
// round-robin to about two blocks per CU, each unit's registers refilled with
// the next unit's codes and block parameters right after use) with the 8-bit
// lane layout above.
template <int EPI, int LPG>
__global__ __launch_bounds__(64 * kStreamWaves) void k_gemv_q8_persist(GemvArgs a) {
  constexpr int EPL = 16, SPAN = 64 * EPL, GROUP = SPAN * LPG;
  extern __shared__ float4 xs4[];  // [KP], zero past K
  __shared__ float s_red[kStreamWaves];
  __shared__ float s_rstd;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;
  const int ng = (K + GROUP - 1) / GROUP;
  const int KP = ng * GROUP;
  const int npairs = (N + 1) / 2;
  const int nw = gridDim.x * kStreamWaves;
  const int gw = blockIdx.x * kStreamWaves + wave;
  const int mine = gw < npairs ? (npairs - 1 - gw) / nw + 1 : 0;
  const int units = mine * ng;
  const uint8_t* Wq = (const uint8_t*)a.W;

  int pos = 0, page = 0, tok = 0;
  if constexpr (EPI == EPI_QKV) {
    pos = a.pos ? a.pos[0] : a.pos_const;
    page = a.kv.page_table ? a.kv.page_table[pos / a.kv.pf] : 0;
  }
  if constexpr (EPI == EPI_EMB) tok = min(max(a.tok[a.tok_col], 0), a.tok_rows - 1);

  u32x4 w0[LPG], w1[LPG];
  uint32_t q0[LPG], q1[LPG];
  auto load_slot = [&](int pair, int g, int i) {
    const int k = min(g * GROUP + i * SPAN + lane * EPL, K - EPL);
    const long long o0 = (long long)min(pair * 2, N - 1) * K + k;
    const long long o1 = (long long)min(pair * 2 + 1, N - 1) * K + k;
    w0[i] = __builtin_nontemporal_load((const u32x4*)(Wq + o0));
    w1[i] = __builtin_nontemporal_load((const u32x4*)(Wq + o1));
    q0[i] = __builtin_nontemporal_load(a.Wq8p + (o0 >> 5));
    q1[i] = __builtin_nontemporal_load(a.Wq8p + (o1 >> 5));
  };
  if (units > 0) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) load_slot(gw, 0, i);
  }

  float rs = 0.f;
  for (int k = tid * 4; k < KP; k += 64 * kStreamWaves * 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < K) {
      v = *(const float4*)(a.x + k);
      if (a.gain) {
        rs += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        const float4 g = *(const float4*)(a.gain + k);
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      }
    }
    xs4[k >> 2] = v;
  }
  if (a.gain) {
    rs = wave_sum(rs);
    if (lane == 0) s_red[wave] = rs;
  }
  __syncthreads();
  if (a.gain && tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) t += s_red[w];
    s_rstd = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
  if (units == 0) return;
  const float rstd = a.gain ? s_rstd : 1.f;

  // epilogue operands, loaded one row pair ahead
  auto load_pre = [&](int pair, float& e0, float& e1) {
    const int r0 = min(pair * 2, N - 1), r1 = min(pair * 2 + 1, N - 1);
    e0 = 0.f;
    e1 = 0.f;
    if constexpr (EPI == EPI_RESID) {
      e0 = a.y[r0];
      e1 = a.y[r1];
    }
    if constexpr (EPI == EPI_EMB) {
      e0 = bf2f(((const uint16_t*)a.emb)[(long long)tok * N + r0]);
      e1 = bf2f(((const uint16_t*)a.emb)[(long long)tok * N + r1]);
    }
    if constexpr (EPI == EPI_QKV) {
      const int dim = (r0 % a.d) % a.hd;
      const float* cs = a.rope + ((long long)pos * (a.hd >> 1) + (dim >> 1)) * 2;
      e0 = cs[0];
      e1 = cs[1];
    }
  };
  float pre0, pre1, nxt0 = 0.f, nxt1 = 0.f;
  load_pre(gw, pre0, pre1);
  float acc0 = 0.f, acc1 = 0.f;

  auto unit = [&](int pair, int g, int npair, int ngrp, bool refill) {
    if (refill) load_pre(npair, nxt0, nxt1);
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int k = g * GROUP + i * SPAN + lane * EPL;
      float xv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 t = xs4[(k + e) >> 2];
        xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
      }
      float sx = 0.f, d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sx += xv[e];
        d0 = fmaf((float)((w0[i][e >> 2] >> (8 * (e & 3))) & 0xffu), xv[e], d0);
        d1 = fmaf((float)((w1[i][e >> 2] >> (8 * (e & 3))) & 0xffu), xv[e], d1);
      }
      acc0 = fmaf(f16_lo(q0[i]), d0, fmaf(f16_hi(q0[i]), sx, acc0));
      acc1 = fmaf(f16_lo(q1[i]), d1, fmaf(f16_hi(q1[i]), sx, acc1));
      if (refill) load_slot(npair, ngrp, i);
    }
    if (g == ng - 1) {
      acc0 = wave_sum(acc0);
      acc1 = wave_sum(acc1);
      if (lane == 0) pair_store<EPI>(a, a.y, pair * 2, acc0 * rstd, acc1 * rstd, pre0, pre1, pos, page);
      acc0 = 0.f;
      acc1 = 0.f;
    }
    if (refill && ngrp == 0) {
      pre0 = nxt0;
      pre1 = nxt1;
    }
  };

  int pair = gw, g = 0;
  for (int u = 0; u < units - 1; ++u) {
    int npair = pair, ngrp = g + 1;
    if (ngrp == ng) {
      ngrp = 0;
      npair += nw;
    }
    unit(pair, g, npair, ngrp, true);
    pair = npair;
    g = ngrp;
  }
  unit(pair, g, pair, g, false);
}

template <int LPG>
static void q8_persist_launch(const GemvArgs& a, int epi, int blocks, hipStream_t s) {
  constexpr int GROUP = 1024 * LPG;
  const size_t lds = (size_t)((a.K + GROUP - 1) / GROUP) * GROUP * sizeof(float);
  const int T = 64 * kStreamWaves;
  switch (epi) {
    case EPI_STORE: k_gemv_q8_persist<EPI_STORE, LPG><<<blocks, T, lds, s>>>(a); break;
    case EPI_RESID: k_gemv_q8_persist<EPI_RESID, LPG><<<blocks, T, lds, s>>>(a); break;
    case EPI_EMB: k_gemv_q8_persist<EPI_EMB, LPG><<<blocks, T, lds, s>>>(a); break;
    case EPI_SWIGLU: k_gemv_q8_persist<EPI_SWIGLU, LPG><<<blocks, T, lds, s>>>(a); break;
    case EPI_QKV: k_gemv_q8_persist<EPI_QKV, LPG><<<blocks, T, lds, s>>>(a); break;
  }
}

template <int SPW>
static void q8_launch(const GemvArgs& a, int epi, int SK, hipStream_t s) {
  const int RG = kStreamWaves / SK;
  dim3 grid(((a.N + 1) / 2 + RG - 1) / RG);
  const size_t lds = (size_t)SK * SPW * 1024 * sizeof(float);
  const int T = 64 * kStreamWaves;
  switch (epi) {
    case EPI_STORE: k_gemv_q8<EPI_STORE, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_RESID: k_gemv_q8<EPI_RESID, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_EMB: k_gemv_q8<EPI_EMB, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_SWIGLU: k_gemv_q8<EPI_SWIGLU, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_QKV: k_gemv_q8<EPI_QKV, SPW><<<grid, T, lds, s>>>(a, SK); break;
  }
}

static int device_cus();

static void gemv_q8(const GemvArgs& a, int B, int epi, hipStream_t s) {
  if (B != 1) throw std::runtime_error("8-bit weights stream one input vector per launch");
  if (a.K % 32 != 0 || a.K < 16) throw std::runtime_error("8-bit weights need K % 32 == 0");
  const int npairs = (a.N + 1) / 2;
  const int nspans = (a.K + 1023) / 1024;
  constexpr int kWaves = 2048;
  if (npairs >= kWaves) {
    // persistent: spans per unit that pad K least (the inputs, padded to whole
    // units, must fit in 64 KB of LDS)
    const int lpg = nspans % 8 == 0 ? 8 : (nspans <= 2 ? 2 : 4);
    const long long kp = (long long)((nspans + lpg - 1) / lpg) * lpg * 1024;
    if (kp * (long long)sizeof(float) <= 65536) {
      const int blocks = std::min((npairs + kStreamWaves - 1) / kStreamWaves, 2 * device_cus());
      if (lpg == 2) q8_persist_launch<2>(a, epi, blocks, s);
      else if (lpg == 4) q8_persist_launch<4>(a, epi, blocks, s);
      else q8_persist_launch<8>(a, epi, blocks, s);
      return;
    }
  }
  // split K inside a block while the grid has fewer than 2048 waves or a wave
  // would need more than 8 spans
  int SK = 1;
  while (SK < kStreamWaves && SK * 2 <= nspans && (npairs * SK < kWaves || (nspans + SK - 1) / SK > 8)) SK *= 2;
  const int need = (nspans + SK - 1) / SK;
  if (need > 8) throw std::runtime_error("8-bit GEMV: rows too long");
  const int spw = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  if ((size_t)SK * spw * 1024 * sizeof(float) > 65536) throw std::runtime_error("8-bit GEMV: inputs exceed LDS");
  if (spw == 1) q8_launch<1>(a, epi, SK, s);
  else if (spw == 2) q8_launch<2>(a, epi, SK, s);
  else if (spw == 4) q8_launch<4>(a, epi, SK, s);
  else q8_launch<8>(a, epi, SK, s);
}

__global__ __launch_bounds__(256) void k_q8_to_f16(const uint8_t* q, const uint32_t* prm, uint16_t* dst, long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const uint32_t pv = prm[i >> 5];
    const float v = fmaf((float)q[i], f16_lo(pv), f16_hi(pv));
    const _Float16 h = (_Float16)v;
    dst[i] = *(const uint16_t*)&h;
  }
}

void launch_q8_to_f16(const uint8_t* q, const uint32_t* params, uint16_t* dst, long long n, hipStream_t s) {
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  k_q8_to_f16<<<(unsigned)blocks, 256, 0, s>>>(q, params, dst, n);
}

// ---------------------------------------------------------------------------
// Batched weight-streaming GEMV on matrix cores (2..16 conversations, bf16
// weights). v_mfma_f32_16x16x32_f16 computes a 16 (rows of W) x 16 (tokens)
// tile: lane l supplies W[row0 + l%16][k0 + 8*(l/16) .. +7] (a 16-byte load)
// and the fp16 normalised input of token l%16 at the same k, and receives
// rows row0 + 4*(l/16) + 0..3 of token l%16 -- so RoPE and SwiGLU pairs stay
// in one lane. Tokens past the batch read zeros. Units are (16-row group,
// K-group of 8 such loads); as in the single-vector kernel each lane refills
// its weight registers with the next unit's data right after use. The
// conversion of a bf16 weight to fp16 is exact in fp16's normal range.
// ---------------------------------------------------------------------------
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t h2pack(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)(*(const uint16_t*)&x) | ((uint32_t)(*(const uint16_t*)&y) << 16);
}
__device__ __forceinline__ h16x8 bf8_to_h16x8(u32x4 v) {
  u32x4 r;
  r.x = h2pack(bf_lo(v.x), bf_hi(v.x));
  r.y = h2pack(bf_lo(v.y), bf_hi(v.y));
  r.z = h2pack(bf_lo(v.z), bf_hi(v.z));
  r.w = h2pack(bf_lo(v.w), bf_hi(v.w));
  return *(const h16x8*)&r;
}


template <int EPI, bool XG, int kMfmaLPG>
__global__ __launch_bounds__(64 * kStreamWaves) void k_gemv_mfma(GemvArgs a, int B, int k_begin, int k_end, int SK) {
  constexpr int GROUP = 32 * kMfmaLPG;  // kMfmaLPG 32-wide K chunks per unit
  extern __shared__ uint16_t xh[];  // fp16 [B][KP], zero past the chunk
  __shared__ float s_red[kStreamWaves][16];
  __shared__ float s_rstd[16];
  __shared__ f32x4v s_part[kStreamWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N;
  const int KC = k_end - k_begin;  // columns handled by this launch
  const int ng = (KC + GROUP - 1) / GROUP;
  const int KP = ng * GROUP;
  const int ngroups = (N + 15) / 16;
  // block = (8 / SK) row groups x SK slices of K; a wave walks its slice
  const int RG = kStreamWaves / SK;
  const int rgl = wave / SK, ks = wave - rgl * SK;
  const int g_lo = ks * ng / SK, g_hi = (ks + 1) * ng / SK;  // this wave's K-groups
  const int nsets = (ngroups + RG - 1) / RG;
  const int my_sets = blockIdx.x < nsets ? (nsets - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int per_set = g_hi - g_lo;
  const int units = my_sets * per_set;
  const uint16_t* Wb = (const uint16_t*)a.W;
  const int tok = lane & 15, quad = lane >> 4;

  // per-token epilogue constants (this lane's token)
  const int tk = min(tok, B - 1);
  int pos_t = 0, page_t = 0, emb_t = 0;
  if constexpr (EPI == EPI_QKV) {
    pos_t = a.pos ? a.pos[tk] : a.pos_const;
    page_t = a.kv.page_table ? a.kv.page_table[tk * a.kv.pt_stride + pos_t / a.kv.pf] : tk;
  }
  if constexpr (EPI == EPI_EMB) emb_t = min(max(a.tok[tk * a.tok_stride + a.tok_col], 0), a.tok_rows - 1);

  auto grp_of = [&](int set) { return min((blockIdx.x + set * (int)gridDim.x) * RG + rgl, ngroups - 1); };
  u32x4 w[kMfmaLPG];
  u32x4 xr[XG ? kMfmaLPG : 1];
  auto load_slot = [&](int grp, int g, int i) {
    const int row = min(grp * 16 + tok, N - 1);
    const int k = min(k_begin + g * GROUP + i * 32 + quad * 8, K - 8);
    w[i] = __builtin_nontemporal_load((const u32x4*)(Wb + (long long)row * K + k));
    if constexpr (XG) xr[i] = *(const u32x4*)(a.x16 + (long long)tk * a.ldx + k);
  };
  if (units > 0) {
#pragma unroll
    for (int i = 0; i < kMfmaLPG; ++i) load_slot(grp_of(0), g_lo, i);
  }

  // prologue, one read of x: LDS gets fp16(gain * x) of [k_begin, k_end),
  // zero past the chunk; the RMSNorm factor of each token scales the dot
  // products in the epilogue. Its statistics come from the producer's partial
  // sums of squares (stat_in, loaded before the inputs so the two overlap), or
  // else from the same pass over x (a launch with a gain covers all of K).
  const bool hand = !XG && a.gain && a.stat_in;
  float st[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = wave + h * kStreamWaves, i = lane + 64 * j;
      st[h][j] = (hand && b < B && i < a.stat_in_n) ? a.stat_in[b * a.stat_in_ld + i] : 0.f;
    }
  float rs[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) rs[b] = 0.f;
  for (int i = tid * 4; i < (XG ? 0 : B * KP); i += 64 * kStreamWaves * 4) {
    const int b = i / KP, k = i - b * KP;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < KC) {
      v = *(const float4*)(a.x + (long long)b * a.ldx + k_begin + k);
      if (a.gain) {
        if (!hand) {
          const float q = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
          for (int bb = 0; bb < 16; ++bb)
            if (bb == b) rs[bb] += q;
        }
        const float4 g = *(const float4*)(a.gain + k_begin + k);
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      }
    }
    *(uint2*)(xh + i) = make_uint2(h2pack(v.x, v.y), h2pack(v.z, v.w));
  }
  if (hand) {
    // partials in a fixed order: lane-strided sums, then the wave reduction
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = wave + h * kStreamWaves;
      float t = (st[h][0] + st[h][1]) + (st[h][2] + st[h][3]);
      for (int i = lane + 256; i < a.stat_in_n; i += 64)
        if (b < B) t += a.stat_in[b * a.stat_in_ld + i];
      t = wave_sum(t);
      if (lane == 0 && b < B) s_rstd[b] = 1.0f / sqrtf(t / (float)K + a.eps);
    }
  } else if (!XG && a.gain) {
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      if (b < B) {
        rs[b] = wave_sum(rs[b]);
        if (lane == 0) s_red[wave][b] = rs[b];
      }
    }
  }
  __syncthreads();
  if (!XG && a.gain && !hand && tid < B) {
    float t = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kStreamWaves; ++w2) t += s_red[w2][tid];
    s_rstd[tid] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
  if (my_sets == 0) return;

  // epilogue operands of a row group (residual / embedding values, RoPE
  // angles), loaded one set ahead and carried
  auto load_pre = [&](int grp, float (&pre)[4]) {
    const int r0 = min(grp * 16 + quad * 4, N - 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) pre[r] = 0.f;
    if constexpr (EPI == EPI_RESID) {
      const float4 v = *(const float4*)(a.y + (long long)tk * a.ldy + r0);
      pre[0] = v.x; pre[1] = v.y; pre[2] = v.z; pre[3] = v.w;
    }
    if constexpr (EPI == EPI_EMB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pre[r] = bf2f(((const uint16_t*)a.emb)[(long long)emb_t * N + r0 + r]);
    }
    if constexpr (EPI == EPI_QKV) {
      const int dim = (r0 % a.d) % a.hd;
      const float* cs = a.rope + ((long long)pos_t * (a.hd >> 1) + (dim >> 1)) * 2;
      pre[0] = cs[0]; pre[1] = cs[1]; pre[2] = cs[2]; pre[3] = cs[3];
    }
  };
  float pre[4], pre_n[4];
  load_pre(grp_of(0), pre);
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
  const float rnorm = (!XG && a.gain) ? s_rstd[tk] : 1.f;  // this lane's token
  const uint16_t* xrow = xh + (long long)tk * KP;
  const bool tok_live = tok < B;

  // units (set, K-group) in order; the steady-state loop always refills, the
  // last unit is peeled so that no load sits behind a data-dependent branch
  auto unit = [&](int set, int g, bool refill) {
    const int grp = grp_of(set);
    int nset = set, ngk = g + 1;
    if (ngk == g_hi) {
      ngk = g_lo;
      ++nset;
    }
    const int ngrp = grp_of(nset);
    if (refill) load_pre(ngrp, pre_n);
#pragma unroll
    for (int i = 0; i < kMfmaLPG; ++i) {
      const int k = g * GROUP + i * 32 + quad * 8;
      u32x4 xv;
      if constexpr (XG) {
        xv = xr[i];
        // chunks past K were read at a clamped address
        if (k_begin + k >= K) xv = u32x4{0, 0, 0, 0};
      } else {
        xv = *(const u32x4*)(xrow + k);
      }
      if (!tok_live) xv = u32x4{0, 0, 0, 0};
      const h16x8 af = bf8_to_h16x8(w[i]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, *(const h16x8*)&xv, acc, 0, 0, 0);
      if (refill) load_slot(ngrp, ngk, i);
      // keep slot order: converting a later slot early would wait for its load
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g == g_hi - 1) {
      // reduce the SK slices of each row group through LDS (fixed order)
      if (SK > 1) {
        s_part[wave][lane] = acc;
        __syncthreads();
        if (ks == 0) {
          for (int j = 1; j < SK; ++j) {
            const f32x4v t = s_part[wave + j][lane];
            acc[0] += t[0]; acc[1] += t[1]; acc[2] += t[2]; acc[3] += t[3];
          }
        }
        __syncthreads();
      }
      const int row = grp * 16 + quad * 4;
      const bool own = (blockIdx.x + set * (int)gridDim.x) * RG + rgl < ngroups;
      if constexpr (EPI == EPI_RESID || EPI == EPI_EMB) {
        if (a.stat_out && ks == 0 && own && k_end == K) {
          // sum of squares of the row group's final outputs (lanes of one token)
          float sq = 0.f;
          if (tok_live && row < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float o = acc[r] * rnorm + pre[r];  // the stored output
              sq = fmaf(o, o, sq);
            }
          }
          sq += __shfl_xor(sq, 16, 64);
          sq += __shfl_xor(sq, 32, 64);
          if (quad == 0 && tok_live) a.stat_out[tok * a.stat_out_ld + grp] = sq;
        }
      }
      if (ks == 0 && tok_live && own && row < N) {
        float* y = a.y + (long long)tok * a.ldy;
        const float v0 = acc[0] * rnorm, v1 = acc[1] * rnorm, v2 = acc[2] * rnorm, v3 = acc[3] * rnorm;
        if constexpr (EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_EMB) {
          *(float4*)(y + row) = make_float4(v0 + pre[0], v1 + pre[1], v2 + pre[2], v3 + pre[3]);
        } else if constexpr (EPI == EPI_SWIGLU) {
          const float o0 = v0 / (1.0f + expf(-v0)) * v1, o1 = v2 / (1.0f + expf(-v2)) * v3;
          *(float2*)(y + (row >> 1)) = make_float2(o0, o1);
          if (a.y16) *(uint32_t*)(a.y16 + (long long)tok * a.ldy + (row >> 1)) = h2pack(o0, o1);
        } else if constexpr (EPI == EPI_QKV) {
          const int part = row / a.d;
          const int rr = row - part * a.d;
          const int head = rr / a.hd, dim = rr - head * a.hd;
          float x0 = v0, x1 = v1, x2 = v2, x3 = v3;
          if (part < 2) {
            x0 = v0 * pre[0] - v1 * pre[1];
            x1 = v0 * pre[1] + v1 * pre[0];
            x2 = v2 * pre[2] - v3 * pre[3];
            x3 = v2 * pre[3] + v3 * pre[2];
          }
          if (part == 0) {
            *(float4*)(y + rr) = make_float4(x0, x1, x2, x3);
          } else {
            const long long off = (long long)page_t * a.kv.page_stride +
                                  ((long long)((a.layer * 2 + part - 1) * a.kv.n_heads + head) * a.kv.pf +
                                   (pos_t % a.kv.pf)) * a.kv.hd + dim;
            if (a.kv_bf16) {
              const uint32_t lo = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
              const uint32_t hi = (uint32_t)f2bf(x2) | ((uint32_t)f2bf(x3) << 16);
              *(uint2*)((uint16_t*)a.kv.base + off) = make_uint2(lo, hi);
            } else {
              *(float4*)((float*)a.kv.base + off) = make_float4(x0, x1, x2, x3);
            }
          }
        }
      }
      acc = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) pre[r] = pre_n[r];
    }
  };
  int set = 0, g = g_lo;
  for (int u = 0; u < units - 1; ++u) {
    unit(set, g, true);
    if (++g == g_hi) {
      g = g_lo;
      ++set;
    }
  }
  unit(set, g, false);
}

static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

// one input vector and fewer row pairs than kSplitWaves: split K over the
// waves of a block (k_gemv_splitk); false when the shape does not qualify
constexpr int kSplitWaves = 2048;

template <bool BF, int SPW, int XP = XP_LOAD>
static void splitk_launch(const GemvArgs& a, int epi, int SK, hipStream_t s) {
  constexpr int SPAN = 64 * WLoad<BF>::EPL;
  const int RG = kStreamWaves / SK;
  const int npairs = (a.N + 1) / 2;
  dim3 grid((npairs + RG - 1) / RG);
  const size_t lds = (size_t)SK * SPW * SPAN * sizeof(float);
  const int T = 64 * kStreamWaves;
  if constexpr (XP != XP_LOAD) {
    k_gemv_splitk<BF, EPI_RESID, SPW, XP><<<grid, T, lds, s>>>(a, SK);
    return;
  }
  switch (epi) {
    case EPI_STORE: k_gemv_splitk<BF, EPI_STORE, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_RESID: k_gemv_splitk<BF, EPI_RESID, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_EMB: k_gemv_splitk<BF, EPI_EMB, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_SWIGLU: k_gemv_splitk<BF, EPI_SWIGLU, SPW><<<grid, T, lds, s>>>(a, SK); break;
    case EPI_QKV: k_gemv_splitk<BF, EPI_QKV, SPW><<<grid, T, lds, s>>>(a, SK); break;
  }
}

// split factor SK and spans per wave of the split-K route, or false when the
// shape does not take it
static bool splitk_plan(const GemvArgs& a, bool bf16, int* SKo, int* spwo) {
  const int target = kSplitWaves;
  const int span = bf16 ? 512 : 256;
  const int npairs = (a.N + 1) / 2;
  const int nspans = (a.K + span - 1) / span;
  if (npairs >= target || a.K % 4 != 0) return false;
  int SK = 1;
  while (SK < kStreamWaves && npairs * SK < target && SK * 2 <= nspans) SK *= 2;
  if (SK < 2) return false;
  const int need = (nspans + SK - 1) / SK;
  const int spw = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  if (need > 8 || (size_t)SK * spw * span * sizeof(float) > 65536) return false;
  *SKo = SK;
  *spwo = spw;
  return true;
}

template <int XP>
static bool gemv_splitk_xp(const GemvArgs& a, int epi, bool bf16, hipStream_t s) {
  int SK, spw;
  if (!splitk_plan(a, bf16, &SK, &spw)) return false;
  if (bf16) {
    if (spw == 1) splitk_launch<true, 1, XP>(a, epi, SK, s);
    else if (spw == 2) splitk_launch<true, 2, XP>(a, epi, SK, s);
    else if (spw == 4) splitk_launch<true, 4, XP>(a, epi, SK, s);
    else splitk_launch<true, 8, XP>(a, epi, SK, s);
  } else {
    if (spw == 1) splitk_launch<false, 1, XP>(a, epi, SK, s);
    else if (spw == 2) splitk_launch<false, 2, XP>(a, epi, SK, s);
    else if (spw == 4) splitk_launch<false, 4, XP>(a, epi, SK, s);
    else splitk_launch<false, 8, XP>(a, epi, SK, s);
  }
  return true;
}

static bool gemv_splitk(const GemvArgs& a, int epi, bool bf16, hipStream_t s) {
  return gemv_splitk_xp<XP_LOAD>(a, epi, bf16, s);
}

// loads per group and padded K of the one-vector persistent route (NB input
// vectors), or false when x does not fit in LDS
template <bool BF>
static bool persist_plan(const GemvArgs& a, int NB, int epi, int* lpgo, size_t* ldso) {
  if ((size_t)NB * a.K * sizeof(float) > 65536) return false;
  constexpr int EPL = WLoad<BF>::EPL;
  const int slots = (a.K + 64 * EPL - 1) / (64 * EPL);
  // QKV maps at most 4 loads per group: the 7B map has 6144 row pairs for
  // 4096 waves, and with more, shorter units the waves that own two pairs keep
  // their loads flowing (18.9 -> 18.3 us per layer; the evenly loaded maps are
  // faster with 8)
  const int lpg = std::min(slots <= 2 ? 2 : (slots <= 4 ? 4 : 8), epi == EPI_QKV ? 4 : 8);
  const int KP = ((a.K + 64 * EPL * lpg - 1) / (64 * EPL * lpg)) * 64 * EPL * lpg;
  const size_t lds_p = (size_t)NB * KP * sizeof(float);
  if (lds_p > 65536) return false;
  *lpgo = lpg;
  *ldso = lds_p;
  return true;
}

// the split-K persistent schedule (KS = 2, 4-load groups): plain or residual
// stores of one input vector whose row pairs fit one per wave pair at two
// blocks per CU and whose K spans at least four groups (the 7B down
// projection: 19.3 -> 18.5 us; the 4096-wide Wo is slower split, 8.4 -> 8.6)
static bool persist_ks_fits(const GemvArgs& a, bool bf16, int epi, size_t* lds) {
  const int group = 64 * (bf16 ? 8 : 4) * 4;
  if (epi != EPI_RESID && epi != EPI_STORE) return false;
  const int npairs = (a.N + 1) / 2;
  const int ng = (a.K + group - 1) / group;
  *lds = (size_t)ng * group * sizeof(float);
  return ng >= 4 && npairs <= 2 * device_cus() * (kStreamWaves / 2) && *lds <= 65536;
}

template <bool BF, int XP>
static void persist_ks_launch(const GemvArgs& a, int epi, size_t lds, hipStream_t s) {
  const dim3 grid(2 * device_cus());
  const int T = 64 * kStreamWaves;
  if (epi == EPI_RESID)
    k_gemv_persist<1, BF, EPI_RESID, 4, XP, 2><<<grid, T, lds, s>>>(a);
  else if constexpr (XP == XP_LOAD)
    k_gemv_persist<1, BF, EPI_STORE, 4, XP, 2><<<grid, T, lds, s>>>(a);
}

template <int NB, bool BF>
static void gemv_dispatch_epi(const GemvArgs& a, int epi, int KC, hipStream_t s) {
  if constexpr (NB == 1) {
    if (gemv_splitk(a, epi, BF, s)) return;
  }
  int lpg;
  size_t lds_p;
  if constexpr (NB == 1) {
    if (persist_ks_fits(a, BF, epi, &lds_p)) {
      persist_ks_launch<BF, XP_LOAD>(a, epi, lds_p, s);
      return;
    }
  }
  if (persist_plan<BF>(a, NB, epi, &lpg, &lds_p)) {
    const int need = ((a.N + 1) / 2 + kStreamWaves - 1) / kStreamWaves;
    // two blocks per CU whenever one per CU would not hold every row pair (the
    // wave-major assignment spreads the pairs over all of them)
    dim3 grid(need > device_cus() ? 2 * device_cus() : need);
    const int T = 64 * kStreamWaves;
#define MOSHI_GP(E, L) k_gemv_persist<NB, BF, E, L><<<grid, T, lds_p, s>>>(a)
#define MOSHI_GPL(E) (lpg == 2 ? MOSHI_GP(E, 2) : (lpg == 4 ? MOSHI_GP(E, 4) : MOSHI_GP(E, 8)))
    switch (epi) {
      case EPI_STORE: MOSHI_GPL(EPI_STORE); break;
      case EPI_RESID: MOSHI_GPL(EPI_RESID); break;
      case EPI_EMB: MOSHI_GPL(EPI_EMB); break;
      case EPI_SWIGLU: MOSHI_GPL(EPI_SWIGLU); break;
      case EPI_QKV: MOSHI_GPL(EPI_QKV); break;
    }
    return;
#undef MOSHI_GPL
#undef MOSHI_GP
  }
  dim3 grid((a.N + kGemvRows - 1) / kGemvRows);
  size_t lds = (size_t)NB * (size_t)KC * sizeof(float);
  switch (epi) {
    case EPI_STORE: k_gemv<NB, BF, EPI_STORE><<<grid, 256, lds, s>>>(a, KC); break;
    case EPI_RESID: k_gemv<NB, BF, EPI_RESID><<<grid, 256, lds, s>>>(a, KC); break;
    case EPI_EMB: k_gemv<NB, BF, EPI_EMB><<<grid, 256, lds, s>>>(a, KC); break;
    case EPI_SWIGLU: k_gemv<NB, BF, EPI_SWIGLU><<<grid, 256, lds, s>>>(a, KC); break;
    case EPI_QKV: k_gemv<NB, BF, EPI_QKV><<<grid, 256, lds, s>>>(a, KC); break;
  }
}

template <bool BF>
static void gemv_dispatch(const GemvArgs& a, int B, int epi, hipStream_t s) {
  constexpr int span = 64 * WLoad<BF>::EPL;
  const int cap = kGemvLdsFloats / B;
  int KC = a.K <= cap ? a.K : (cap / span) * span;
  switch (B) {
    case 1: gemv_dispatch_epi<1, BF>(a, epi, KC, s); break;
    case 2: gemv_dispatch_epi<2, BF>(a, epi, KC, s); break;
    case 3: gemv_dispatch_epi<3, BF>(a, epi, KC, s); break;
    case 4: gemv_dispatch_epi<4, BF>(a, epi, KC, s); break;
    case 5: gemv_dispatch_epi<5, BF>(a, epi, KC, s); break;
    case 6: gemv_dispatch_epi<6, BF>(a, epi, KC, s); break;
    case 7: gemv_dispatch_epi<7, BF>(a, epi, KC, s); break;
    case 8: gemv_dispatch_epi<8, BF>(a, epi, KC, s); break;
  }
}

template <int EPI, int kMfmaLPG>
static void gemv_mfma_launch_lpg(const GemvArgs& a, int B, hipStream_t s) {
  constexpr int GROUP = 32 * kMfmaLPG;
  const int ngroups = (a.N + 15) / 16;
  // split K inside a block until the grid has about 2048 waves
  int SK = 1;
  const int ng_launch = (std::min(a.K, (65536 / (2 * B)) / GROUP * GROUP) + GROUP - 1) / GROUP;
  // finest sets (one row group per block) balance the per-CU byte counts best
  while (SK < kStreamWaves && SK * 2 <= ng_launch) SK *= 2;
  const int RG = kStreamWaves / SK;
  const int nsets = (ngroups + RG - 1) / RG;
  dim3 grid(std::min(nsets, 2 * device_cus()));
  const int T = 64 * kStreamWaves;
  // the fp16 inputs of one launch must fit in 64 KB of LDS: long rows (the
  // residual down projection) run as several launches over K ranges, each
  // adding its partial product into y
  const int cap = (65536 / (2 * B)) / GROUP * GROUP;
  if (a.K <= cap || EPI != EPI_RESID) {
    const int KP = (a.K + GROUP - 1) / GROUP * GROUP;
    k_gemv_mfma<EPI, false, kMfmaLPG><<<grid, T, (size_t)B * KP * 2, s>>>(a, B, 0, a.K, SK);
    return;
  }
  if (a.x16 && !a.gain) {
    // one launch that reads the fp16 inputs directly (L2-resident) instead of LDS
    const int ng_all = (a.K + GROUP - 1) / GROUP;
    int SKx = 1;
    while (SKx < kStreamWaves && SKx * 2 <= ng_all) SKx *= 2;
    const int RGx = kStreamWaves / SKx;
    const int nsx = (ngroups + RGx - 1) / RGx;
    k_gemv_mfma<EPI, true, kMfmaLPG><<<dim3(std::min(nsx, 2 * device_cus())), T, 0, s>>>(a, B, 0, a.K, SKx);
    return;
  }
  const int passes = (a.K + cap - 1) / cap;
  const int step = ((a.K + passes - 1) / passes + 7) / 8 * 8;
  for (int k0 = 0; k0 < a.K; k0 += step) {
    const int k1 = std::min(a.K, k0 + step);
    const int KP = (k1 - k0 + GROUP - 1) / GROUP * GROUP;
    k_gemv_mfma<EPI, false, kMfmaLPG><<<grid, T, (size_t)B * KP * 2, s>>>(a, B, k0, k1, SK);
  }
}

template <int EPI>
static void gemv_mfma_launch(const GemvArgs& a, int B, hipStream_t s) {
  // maps with few 16-row groups (the depth model's) take 128-wide K groups,
  // so that more waves share each row group's K: batch-8 step 8.91 -> 8.70 ms
  // (64-wide: 8.76 ms; 128-wide for every map: 8.76 ms)
  if ((a.N + 15) / 16 < 256)
    gemv_mfma_launch_lpg<EPI, 4>(a, B, s);
  else
    gemv_mfma_launch_lpg<EPI, 8>(a, B, s);
}

static void no_stats(const GemvArgs& a) {
  if (a.stat_in || a.stat_out) throw std::runtime_error("RMSNorm statistics hand-off needs the batched matrix-core GEMV");
}

void launch_gemv(const GemvArgs& a, int B, int epi, bool bf16, hipStream_t s) {
  if (a.Wq8p) {
    if (a.stat_in || a.stat_out) throw std::runtime_error("8-bit GEMV takes no statistics hand-off");
    gemv_q8(a, B, epi, s);
    return;
  }
  // batched bf16: matrix cores, when the fp16 inputs fit in LDS
  if (bf16 && B >= 2 && B <= 16 && (size_t)B * ((a.K + 255) / 256 * 256) * 2 <= 65536 * 3 && a.K % 8 == 0 &&
      a.N % 4 == 0) {
    const int cap = (65536 / (2 * B)) / 256 * 256;
    if (a.K <= cap || epi == EPI_RESID) {
      switch (epi) {
        case EPI_STORE: gemv_mfma_launch<EPI_STORE>(a, B, s); break;
        case EPI_RESID: gemv_mfma_launch<EPI_RESID>(a, B, s); break;
        case EPI_EMB: gemv_mfma_launch<EPI_EMB>(a, B, s); break;
        case EPI_SWIGLU: gemv_mfma_launch<EPI_SWIGLU>(a, B, s); break;
        case EPI_QKV: gemv_mfma_launch<EPI_QKV>(a, B, s); break;
      }
      return;
    }
  }
  no_stats(a);
  if (bf16)
    gemv_dispatch<true>(a, B, epi, s);
  else
    gemv_dispatch<false>(a, B, epi, s);
}

// ---------------------------------------------------------------------------
// Causal decode attention, split over key ranges (flash-decode). Block
// (split, head, conversation) owns keys [P*split/NS, P*(split+1)/NS) of the
// P = pos+1 cached positions (at most kAttnMaxKeys). A group of HD/EPL lanes
// handles one key (each lane holds EPL query values): the block first scores
// all its keys into LDS, takes the softmax statistics with block reductions,
// then accumulates P*V in the same lane layout. With one split the block
// writes the normalised output; otherwise it writes (o, max, sum) and a second
// kernel merges the splits in split order, so results do not depend on timing.
// ---------------------------------------------------------------------------
constexpr int kAttnMaxKeys = 512;

template <bool KBF, int HD>
__device__ __forceinline__ void load_kv16(const void* base, long long off, float (&v)[KBF ? 8 : 4]) {
  if constexpr (KBF) {
    u32x4 t = *(const u32x4*)((const uint16_t*)base + off);
    v[0] = bf_lo(t.x); v[1] = bf_hi(t.x); v[2] = bf_lo(t.y); v[3] = bf_hi(t.y);
    v[4] = bf_lo(t.z); v[5] = bf_hi(t.z); v[6] = bf_lo(t.w); v[7] = bf_hi(t.w);
  } else {
    f32x4 t = *(const f32x4*)((const float*)base + off);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
}

__device__ __forceinline__ float block_max256(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum256(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <bool KBF, int HD>
__global__ __launch_bounds__(256) void k_attn_split(AttnArgs a) {
  constexpr int EPL = KBF ? 8 : 4;
  constexpr int G = HD / EPL;   // lanes per key
  constexpr int KPW = 64 / G;   // keys per wave per pass
  constexpr int KPB = 4 * KPW;  // keys per block per pass
  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z, H = gridDim.y, NS = gridDim.x;
  const int P = (a.pos ? a.pos[b] : a.pos_const) + 1;
  const int k0 = (int)((long long)P * sp / NS), k1 = (int)((long long)P * (sp + 1) / NS);
  const int n = k1 - k0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane % G, g = lane / G;
  __shared__ float sc[kAttnMaxKeys];
  __shared__ float so[KPB * HD];
  __shared__ float red[4];

  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = a.q[(long long)b * a.ldq + h * HD + li * EPL + e] * a.scale;

  // scores
#pragma unroll 4
  for (int base = k0 + wave * KPW; base < k1; base += KPB) {
    const int key = base + g;
    float d = 0.f;
    if (key < k1) {
      float kf[EPL];
      load_kv16<KBF, HD>(a.kv.base, a.kv.offset(b, a.layer, 0, h, key) + li * EPL, kf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qv[e], kf[e], d);
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
    if (key < k1 && li == 0) sc[key - k0] = d;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int i = tid; i < n; i += 256) m = fmaxf(m, sc[i]);
  m = block_max256(m, red);
  float l = 0.f;
  for (int i = tid; i < n; i += 256) {
    const float p = expf(sc[i] - m);
    sc[i] = p;
    l += p;
  }
  l = block_sum256(l, red);  // contains the barrier that publishes sc

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int base = k0 + wave * KPW; base < k1; base += KPB) {
    const int key = base + g;
    if (key < k1) {
      const float p = sc[key - k0];
      float vf[EPL];
      load_kv16<KBF, HD>(a.kv.base, a.kv.offset(b, a.layer, 1, h, key) + li * EPL, vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) so[(wave * KPW + g) * HD + li * EPL + e] = acc[e];
  __syncthreads();
  if (tid < HD) {
    float o = 0.f;
#pragma unroll 4
    for (int i = 0; i < KPB; ++i) o += so[i * HD + tid];
    if (NS == 1) {
      a.out[(long long)b * a.ldo + h * HD + tid] = o / l;
    } else {
      float* part = a.part + ((long long)(b * H + h) * NS + sp) * (HD + 2);
      part[tid] = o;
      if (tid == 0) {
        part[HD] = m;
        part[HD + 1] = l;
      }
    }
  }
}

// Decode attention over the paged temporal cache. Block (split, head,
// conversation) owns keys [P*split/NS, P*(split+1)/NS) of the P = pos+1
// positions; NS is chosen so that the grid has about 128 blocks. The
// block looks its page ids up once, then walks its keys in passes of 4*KPW;
// each group of G lanes keeps its own online-softmax state (running max, sum,
// P*V accumulator) over the keys it saw, with K and V of a chunk of passes
// requested together, so the key loop has no block barriers. The 4*KPW states
// are merged through LDS at the end; with NS > 1 the block writes (o, max, sum)
// and k_attn_merge combines the splits in split order.
constexpr int kAttnWaves = 4;
constexpr int kAttnPasses = 8;
constexpr int kMaxAttnSplits = 16;

template <bool KBF, int HD>
__global__ __launch_bounds__(64 * kAttnWaves) void k_attn_range(AttnArgs a) {
  constexpr int EPL = KBF ? 8 : 4;
  constexpr int ESZ = KBF ? 2 : 4;
  constexpr int G = HD / EPL;
  constexpr int KPW = 64 / G;
  constexpr int KPB = kAttnWaves * KPW;
  constexpr int NST = KPB;  // lane-group states
  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z, NS = gridDim.x, H = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane % G, g = lane / G;
  const int P = a.pos[b] + 1;
  const int k0 = (int)((long long)P * sp / NS), k1 = (int)((long long)P * (sp + 1) / NS);
  const KvView& kv = a.kv;
  __shared__ int pages[kMaxPagesPerConv];
  __shared__ float st_m[NST], st_l[NST];
  __shared__ float st_o[NST * HD];
  const int pg0 = k0 / kv.pf, pg1 = k1 > k0 ? (k1 - 1) / kv.pf : pg0;
  for (int i = pg0 + tid; i <= pg1; i += 64 * kAttnWaves) pages[i - pg0] = kv.page_table[b * kv.pt_stride + i];

  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = a.q[(long long)b * a.ldq + h * HD + li * EPL + e] * a.scale;
  __syncthreads();

  const long long head_off = (long long)((a.layer * 2) * kv.n_heads + h) * kv.pf * kv.hd;
  const long long v_off = (long long)kv.n_heads * kv.pf * kv.hd * ESZ;  // K block -> V block, bytes
  float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  for (int c0 = k0; c0 < k1; c0 += KPB * kAttnPasses) {
    u32x4 kr[kAttnPasses], vr[kAttnPasses];
#pragma unroll
    for (int i = 0; i < kAttnPasses; ++i) {
      const int key = min(c0 + i * KPB + wave * KPW + g, k1 - 1);
      const long long off = (long long)pages[key / kv.pf - pg0] * kv.page_stride + head_off +
                            (long long)(key % kv.pf) * kv.hd + li * EPL;
      const char* base = (const char*)kv.base + off * ESZ;
      kr[i] = *(const u32x4*)base;
      vr[i] = *(const u32x4*)(base + v_off);
    }
    asm volatile("" ::: "memory");  // keep every K and V request ahead of the math
    float sc[kAttnPasses];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < kAttnPasses; ++i) {
      float kf[EPL];
      unpack16<KBF>(kr[i], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qv[e], kf[e], d);
#pragma unroll
      for (int o = G / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
      sc[i] = (c0 + i * KPB + wave * KPW + g < k1) ? d : -INFINITY;
      cmax = fmaxf(cmax, sc[i]);
    }
    const float mn = fmaxf(m, cmax);
    if (mn != -INFINITY) {
      const float alpha = expf(m - mn);  // m = -inf -> 0
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
      for (int i = 0; i < kAttnPasses; ++i) {
        const float p = expf(sc[i] - mn);  // keys outside the range -> 0
        l += p;
        float vf[EPL];
        unpack16<KBF>(vr[i], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
      }
      m = mn;
    }
  }
  const int st = wave * KPW + g;
  if (li == 0) {
    st_m[st] = m;
    st_l[st] = l;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) st_o[st * HD + li * EPL + e] = acc[e];
  __syncthreads();
  if (tid < HD) {
    float M = -INFINITY;
    for (int i = 0; i < NST; ++i) M = fmaxf(M, st_m[i]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
      for (int i = 0; i < NST; ++i) {
        const float w = st_m[i] == -INFINITY ? 0.f : expf(st_m[i] - M);
        L = fmaf(w, st_l[i], L);
        o = fmaf(w, st_o[i * HD + tid], o);
      }
    }
    if (NS == 1) {
      a.out[(long long)b * a.ldo + h * HD + tid] = o / L;
    } else {
      float* part = a.part + ((long long)(b * H + h) * NS + sp) * (HD + 2);
      part[tid] = o;
      if (tid == 0) {
        part[HD] = M;
        part[HD + 1] = L;
      }
    }
  }
}

template <int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(AttnArgs a, int NS) {
  const int h = blockIdx.x, b = blockIdx.y, H = gridDim.x, t = threadIdx.x;
  const float* part = a.part + (long long)(b * H + h) * NS * (HD + 2);
  float M = -INFINITY;
  for (int i = 0; i < NS; ++i) M = fmaxf(M, part[i * (HD + 2) + HD]);
  float L = 0.f, o = 0.f;
  for (int i = 0; i < NS; ++i) {
    const float* pi = part + i * (HD + 2);
    const float w = pi[HD + 1] > 0.f ? expf(pi[HD] - M) : 0.f;
    L = fmaf(w, pi[HD + 1], L);
    o = fmaf(w, pi[t], o);
  }
  a.out[(long long)b * a.ldo + h * HD + t] = o / L;
}

// Depth attention: at most kDepthAttnKeys keys of this frame's positions
// (fp32 cache), one wave per (head, conversation), lane = head dimension
// (hd <= 64). q, K and V are requested together, so the kernel waits on
// memory once; softmax with max subtraction.
constexpr int kDepthAttnKeys = 16;

template <int NK>
__global__ __launch_bounds__(64) void k_attn_depth(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int P = (a.pos ? a.pos[b] : a.pos_const) + 1;
  float o[1];
  depth_attn_heads<NK, 1>(a.q + (long long)b * a.ldq, a.kv, b, a.layer, h, 0, gridDim.x, P, a.scale, lane, o);
  if (lane < a.kv.hd) a.out[(long long)b * a.ldo + h * a.kv.hd + lane] = o[0];
}

static bool depth_attn_ok(const AttnArgs& a, int hd, bool kv_bf16) {
  return !a.kv.page_table && !a.pos && !kv_bf16 && a.pos_const < kDepthAttnKeys && a.pos_const < a.kv.pf &&
         hd <= 64 && a.kv.hd == hd;
}

// temporal cache: about half a block per CU over (split, head, conversation);
// at batch 1 and ~500 keys, 4 splits of 32 heads beat 8 (4.11 vs 4.16 ms per
// frame) and 16-wave blocks without splits are no better
static int attn_range_splits(const AttnArgs& a, int B, int H) {
  return std::max(1, std::min(std::min(a.max_splits, kMaxAttnSplits), 128 / (B * H)));
}

// key-range attention over the paged cache; the splits are merged by
// k_attn_merge unless `merge` is false (the consumer merges them)
static void launch_attn_range(const AttnArgs& a, int B, int H, int hd, bool kv_bf16, int NS, bool merge,
                              hipStream_t s) {
  dim3 grid(NS, H, B);
  const int T = 64 * kAttnWaves;
#define MOSHI_AR(KB, HDV)                                                  \
  do {                                                                     \
    k_attn_range<KB, HDV><<<grid, T, 0, s>>>(a);                           \
    if (NS > 1 && merge) k_attn_merge<HDV><<<dim3(H, B), HDV, 0, s>>>(a, NS); \
  } while (0)
  if (kv_bf16) {
    if (hd == 32) MOSHI_AR(true, 32);
    else if (hd == 64) MOSHI_AR(true, 64);
    else MOSHI_AR(true, 128);
  } else {
    if (hd == 32) MOSHI_AR(false, 32);
    else if (hd == 64) MOSHI_AR(false, 64);
    else MOSHI_AR(false, 128);
  }
#undef MOSHI_AR
}

void launch_attn_decode(const AttnArgs& a, int B, int H, int hd, bool kv_bf16, hipStream_t s) {
  if (depth_attn_ok(a, hd, kv_bf16)) {
    if (a.pos_const < 8)
      k_attn_depth<8><<<dim3(H, B), 64, 0, s>>>(a);
    else
      k_attn_depth<16><<<dim3(H, B), 64, 0, s>>>(a);
    return;
  }
  if (a.kv.page_table && a.pos) {
    launch_attn_range(a, B, H, hd, kv_bf16, attn_range_splits(a, B, H), true, s);
    return;
  }
  const int NS = a.max_splits;
  dim3 grid(NS, H, B);
#define MOSHI_ATTN(KB, HDV)                                                   \
  do {                                                                        \
    k_attn_split<KB, HDV><<<grid, 256, 0, s>>>(a);                            \
    if (NS > 1) k_attn_merge<HDV><<<dim3(H, B), HDV, 0, s>>>(a, NS);          \
  } while (0)
  if (kv_bf16) {
    if (hd == 32) MOSHI_ATTN(true, 32);
    else if (hd == 64) MOSHI_ATTN(true, 64);
    else MOSHI_ATTN(true, 128);
  } else {
    if (hd == 32) MOSHI_ATTN(false, 32);
    else if (hd == 64) MOSHI_ATTN(false, 64);
    else MOSHI_ATTN(false, 128);
  }
#undef MOSHI_ATTN
}

bool launch_attn_wo(const AttnArgs& at, int B, int H, int hd, bool kv_bf16, GemvArgs wo, bool bf16, hipStream_t s) {
  if (B != 1 || wo.Wq8p || wo.stat_in || wo.stat_out || wo.gain || wo.K != H * hd || hd % 4 != 0) return false;
  int SK, spw, lpg;
  size_t lds;
  if (depth_attn_ok(at, hd, kv_bf16)) {
    // the whole depth attention in the split-K prologue
    if (!splitk_plan(wo, bf16, &SK, &spw)) return false;
    wo.attn_q = at.q;
    wo.attn_scale = at.scale;
    wo.kv = at.kv;
    wo.layer = at.layer;
    wo.pos_const = at.pos_const;
    wo.hd = hd;
    return gemv_splitk_xp<XP_ATTN>(wo, EPI_RESID, bf16, s);
  }
  if (!at.kv.page_table || !at.pos || (hd != 32 && hd != 64 && hd != 128)) return false;
  const int NS = attn_range_splits(at, B, H);
  if (NS < 2 || NS > kMergeMaxSplits) return false;
  wo.merge_part = at.part;
  wo.merge_ns = NS;
  wo.hd = hd;
  const bool sk = splitk_plan(wo, bf16, &SK, &spw);
  size_t lds_ks = 0;
  const bool kq = !sk && persist_ks_fits(wo, bf16, EPI_RESID, &lds_ks);
  const bool ps = bf16 ? persist_plan<true>(wo, 1, EPI_RESID, &lpg, &lds) : persist_plan<false>(wo, 1, EPI_RESID, &lpg, &lds);
  if (!sk && !kq && !ps) return false;
  launch_attn_range(at, B, H, hd, kv_bf16, NS, false, s);
  if (sk) return gemv_splitk_xp<XP_MERGE>(wo, EPI_RESID, bf16, s);
  if (kq) {
    if (bf16)
      persist_ks_launch<true, XP_MERGE>(wo, EPI_RESID, lds_ks, s);
    else
      persist_ks_launch<false, XP_MERGE>(wo, EPI_RESID, lds_ks, s);
    return true;
  }
  const int need = ((wo.N + 1) / 2 + kStreamWaves - 1) / kStreamWaves;
  dim3 grid(need > device_cus() ? 2 * device_cus() : need);
  const int T = 64 * kStreamWaves;
#define MOSHI_GM(BFV, L) k_gemv_persist<1, BFV, EPI_RESID, L, XP_MERGE><<<grid, T, lds, s>>>(wo)
  if (bf16) {
    if (lpg == 2) MOSHI_GM(true, 2);
    else if (lpg == 4) MOSHI_GM(true, 4);
    else MOSHI_GM(true, 8);
  } else {
    if (lpg == 2) MOSHI_GM(false, 2);
    else if (lpg == 4) MOSHI_GM(false, 4);
    else MOSHI_GM(false, 8);
  }
#undef MOSHI_GM
  return true;
}

// ---------------------------------------------------------------------------
// Temporal input: the sum of the 17 sub-streams' embedding rows of the
// previous frame (walkthrough, "使用 RQ-Transformer ...": the input of step s
// is the sum of K learnt embedding tables of V_{s-1}).
// ---------------------------------------------------------------------------
template <bool BF>
__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
  const int b = blockIdx.y;
  const int i = min(blockIdx.x * 256 + threadIdx.x, a.d - 1);
  const bool live = blockIdx.x * 256 + threadIdx.x < a.d;
  int t[kStreams];
#pragma unroll
  for (int k = 0; k < kStreams; ++k) t[k] = a.frames[b * kStreams + k];
  float v[kStreams];
#pragma unroll
  for (int k = 0; k < kStreams; ++k) {
    int tk = t[k];
    if (tk < 0 || tk >= a.rows[k]) {
      if (i == 0) atomicOr(a.err, 1);
      tk = a.rows[k] - 1;
    }
    const long long idx = (a.row0[k] + tk) * (long long)a.d + i;
    v[k] = BF ? bf2f(((const uint16_t*)a.table)[idx]) : ((const float*)a.table)[idx];
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kStreams; ++k) s += v[k];
  if (live) a.h[(long long)b * a.d + i] = s;
  if (a.stat_out) {
    __shared__ float red[4];
    const float sq = wave_sum(live ? s * s : 0.f);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
    __syncthreads();
    if (threadIdx.x == 0) a.stat_out[b * a.stat_ld + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

void launch_embed(const EmbedArgs& a, int B, bool bf16, hipStream_t s) {
  dim3 grid((a.d + 255) / 256, B);
  if (bf16)
    k_embed<true><<<grid, 256, 0, s>>>(a);
  else
    k_embed<false><<<grid, 256, 0, s>>>(a);
}

// ---------------------------------------------------------------------------
// Greedy choice: argmax with the lowest index winning ties.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// Counter-based generator for temperature sampling: Philox4x64-10 (Salmon et
// al., "Parallel random numbers: as easy as 1, 2, 3", SC'11), ten rounds of two
// 64 x 64 -> 128-bit products with the key bumped by Weyl constants in between.
__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(c[0], M0), lo0 = c[0] * M0;
    const uint64_t hi1 = __umul64hi(c[2], M1), lo1 = c[2] * M1;
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Gumbel noise -log(-log u) of a generator word: u = (2 (x >> 41) + 1) 2^-24,
// exact in float32 and inside (0, 1)
__device__ __forceinline__ float gumbel_of(uint64_t x) {
  const float u = (float)(2u * (uint32_t)(x >> 41) + 1u) * 0x1p-24f;
  return -logf(-logf(u));
}

struct Sampler {
  float temp;
  uint64_t seed;
};
__device__ __forceinline__ Sampler sampler_of(const ArgmaxArgs& a) {
  Sampler s{0.f, 0};
  if (a.samp) {
    s.temp = __int_as_float(a.samp[a.slot == 0 ? 0 : 1]);
    s.seed = (uint64_t)(uint32_t)a.samp[2] | ((uint64_t)(uint32_t)a.samp[3] << 32);
  }
  return s;
}
// the noise of element i of a draw: counter (i / 4, position, conversation,
// slot), word i % 4, key (seed, 0)
__device__ __forceinline__ float gumbel_at(int i, int pos, int b, int slot, uint64_t seed) {
  uint64_t c[4] = {(uint64_t)(i >> 2), (uint64_t)pos, (uint64_t)b, (uint64_t)slot};
  philox4x64_10(c, seed, 0);
  return gumbel_of(c[i & 3]);
}

// Zero-shot TTS text control (walkthrough appendix C, TTS mode, Fig. 9): inside
// a word its next token is fed without consulting the model; otherwise the
// argmax with a bonus on PAD while the running PAD ratio is under the target
// decides: PAD or EPAD is kept, any other choice starts the next word (PAD once
// the text is used up). best/bi: the plain argmax of the logits l.
__device__ int tts_choose(const ArgmaxArgs& a, int* ctl, const float* l, float best, int bi, Sampler sm) {
  const int b = blockIdx.x;
  const int n = ctl[0], pad = ctl[4], epad = ctl[5];
  int cur = ctl[1], n_pad = ctl[2], n_steps = ctl[3];
  const float target = __int_as_float(ctl[6]), bonus = __int_as_float(ctl[7]);
  const int* tok = a.tts_tok + (long long)b * a.tts_cap;
  const int* wstart = a.tts_start + (long long)b * a.tts_cap;
  int t;
  if (cur > 0 && cur < n && !wstart[cur]) {
    t = tok[cur++];
  } else {
    if ((float)n_pad < target * (float)max(n_steps, 1)) {
      // PAD's score with the bonus on its logit (the bonus is >= 0, so comparing
      // it with the block's best is the argmax over the boosted logits)
      const float boosted = l[pad] + bonus;
      const float score = sm.temp > 0.f ? boosted / sm.temp + gumbel_at(pad, a.pos[b], b, 0, sm.seed) : boosted;
      better(best, bi, score, pad);
    }
    if (bi == pad || bi == epad) t = bi;
    else if (cur < n) t = tok[cur++];
    else t = pad;
  }
  ctl[1] = cur;
  ctl[2] = n_pad + (t == pad ? 1 : 0);
  ctl[3] = n_steps + 1;
  return t;
}

__global__ __launch_bounds__(1024) void k_argmax(ArgmaxArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* l = a.logits + (long long)b * a.ld;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const Sampler sm = sampler_of(a);
  // indices increase within a thread, so a strict '>' keeps the lowest index of
  // equal values
  if (sm.temp > 0.f) {
    // temperature draw, Gumbel-max form: argmax of l / T + Gumbel noise; a thread
    // takes the 4 elements of one generator block at a time
    const int pos = a.pos[b];
    for (int g4 = tid; g4 * 4 < a.n; g4 += 1024) {
      uint64_t c[4] = {(uint64_t)g4, (uint64_t)pos, (uint64_t)b, (uint64_t)a.slot};
      philox4x64_10(c, sm.seed, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = g4 * 4 + w;
        if (i < a.n) {
          const float v = l[i] / sm.temp + gumbel_of(c[w]);
          if (v > bv) {
            bv = v;
            bi = i;
          }
        }
      }
    }
  }
  // greedy: 8 independent loads in flight per thread
  for (int base = 0; sm.temp <= 0.f && base < a.n; base += 1024 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 1024 + tid;
      v[u] = i < a.n ? l[i] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 1024 + tid;
      if (v[u] > bv) {
        bv = v[u];
        bi = i;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) better(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
  __shared__ float sv[16];
  __shared__ int si[16];
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w) better(bv, bi, sv[w], si[w]);
    int own = (bi == 0x7fffffff) ? 0 : bi;
    int* ctl = a.tts_ctl ? a.tts_ctl + b * kTtsCtl : nullptr;
    if (ctl && ctl[0] > 0) own = tts_choose(a, ctl, l, bv, own, sm);
    if (a.pos[b] < a.start) own = a.pad_id;
    a.out_tok[b * a.stride + a.col] = own;
    const int f = *a.has_force ? a.force[b * a.stride + a.col] : -1;
    a.cur_tok[b * a.stride + a.col] = f >= 0 ? f : own;
  }
}

void launch_argmax(const ArgmaxArgs& a, int B, hipStream_t s) { k_argmax<<<B, 1024, 0, s>>>(a); }

// ---------------------------------------------------------------------------
// End of a frame: V_s = (Moshi's slots fed forward) ++ (user's slots) becomes
// the next input; the position advances.
// ---------------------------------------------------------------------------
__global__ void k_advance(AdvanceArgs a, int B) {
  const int t = threadIdx.x;
  if (t < B * kStreams) {
    const int b = t / kStreams, k = t - b * kStreams;
    const int hi = k == 0 ? a.pad_text : a.pad_audio;
    int v;
    if (k >= kSlots) {
      v = a.user_cur ? a.user_cur[b * 8 + (k - kSlots)] : a.user[b * 8 + (k - kSlots)];
    } else {
      const int f = *a.has_force ? a.force[b * kSlots + k] : -1;
      if (f >= 0) v = f;
      else if (a.text_only && k >= 1) v = a.pad_audio;
      else v = a.cur_tok[b * kSlots + k];
    }
    if (v < 0 || v > hi) {
      atomicOr(a.err, 1);
      v = hi;
    }
    if (a.text_only && k >= 1 && k < kSlots) a.out_tok[b * kSlots + k] = v;
    a.prev[b * kStreams + k] = v;
  }
  __syncthreads();
  if (t < B) a.pos[t] += 1;
}

void launch_advance(const AdvanceArgs& a, int B, hipStream_t s) { k_advance<<<1, 256, 0, s>>>(a, B); }

// ---------------------------------------------------------------------------
// Weight repack: float32 rows -> destination rows r*mult + add (float32 or bf16).
// ---------------------------------------------------------------------------
__global__ void k_convert(const float* src, long long rows, int cols, void* dst, int bf, long long mult,
                          long long add) {
  const long long total = rows * cols;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long r = i / cols, c = i - r * cols;
    const long long o = (r * mult + add) * cols + c;
    if (bf)
      ((uint16_t*)dst)[o] = f2bf(src[i]);
    else
      ((float*)dst)[o] = src[i];
  }
}

void launch_convert(const float* src, long long rows, int cols, void* dst, bool bf16, long long mult, long long add,
                    hipStream_t s) {
  long long total = rows * cols;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  k_convert<<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, dst, bf16 ? 1 : 0, mult, add);
}

}  // namespace moshi
