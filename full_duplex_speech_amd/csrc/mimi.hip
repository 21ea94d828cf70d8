// Bottleneck Transformer of the Mimi codec (walkthrough of the Moshi report,
// section "基于 Transformer 的瓶颈"; notes page section 3a): 8 pre-norm layers of
// width 512 with 8 heads, RoPE, causal attention limited to the last 250
// frames, a GELU MLP of width 2048 and LayerScale on both residual branches.
// Float32 throughout. Per layer: LayerNorm -> QKV GEMM with RoPE fused into its
// epilogue -> sliding-window attention -> Wo GEMM adding scale1 * out to the
// stream -> LayerNorm -> W1 GEMM with GELU -> W2 GEMM adding scale2 * out.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/moshi.h"
#include "gemm_f32.h"

namespace {

using namespace moshi_f32;

constexpr int kD = 512, kH = 8, kHD = 64, kF = 2048;
constexpr int kQT = 64;     // queries per attention block (one wave, lane = query)
constexpr int kKC = 32;     // keys per LDS chunk

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// y = (x - mean) / sqrt(var + eps) * g + b over rows of 512; one wave per row
__global__ __launch_bounds__(256) void k_layer_norm(const float* x, const float* g, const float* b, float* y,
                                                    int M) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const float* r = x + (long long)m * kD;
  float v[8];
  const float4 a = *(const float4*)(r + lane * 4), c = *(const float4*)(r + 256 + lane * 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  const float mu = wsum(s) / (float)kD;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) q = fmaf(v[i] - mu, v[i] - mu, q);
  const float rstd = 1.0f / sqrtf(wsum(q) / (float)kD + 1e-5f);
  float* o = y + (long long)m * kD;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = h * 256 + lane * 4;
    const float4 gg = *(const float4*)(g + k), bb = *(const float4*)(b + k);
    *(float4*)(o + k) = make_float4((v[4 * h] - mu) * rstd * gg.x + bb.x, (v[4 * h + 1] - mu) * rstd * gg.y + bb.y,
                                    (v[4 * h + 2] - mu) * rstd * gg.z + bb.z, (v[4 * h + 3] - mu) * rstd * gg.w + bb.w);
  }
}

// RoPE table [S][hd/2] of (cos, sin) of pos * 10000^(-2i/hd), computed in double
__global__ void k_rope_table64(float* t, int S, int hd) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int half = hd / 2;
  if (i >= S * half) return;
  const int pos = i / half, j = i - pos * half;
  const double ang = (double)pos * pow(10000.0, -2.0 * j / hd);
  t[2 * i] = (float)cos(ang);
  t[2 * i + 1] = (float)sin(ang);
}

// Sliding-window causal attention. Block (query tile, head, sequence), one wave:
// lane = query t (its q scaled by 1/sqrt(hd) and its output in registers); keys
// max(0, t0 - W + 1) .. t0 + 63 pass through LDS in chunks of 32. Per chunk the
// lane scores its allowed keys, rescales its running output once to the new
// maximum, then accumulates the chunk's values.
__global__ __launch_bounds__(64) void k_window_attn(const float* qkv, float* out, int S, int window) {
  __shared__ float4 ks[kKC][kHD / 4];
  __shared__ float4 vs[kKC][kHD / 4];
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * kQT, h = blockIdx.y, bseq = blockIdx.z;
  const int t = t0 + lane;
  const bool live = t < S;
  const long long row0 = (long long)bseq * S;
  const int ld = 3 * kD;
  float q[kHD], o[kHD];
  const float scale = 0.125f;  // 1 / sqrt(64)
  {
    const float* qp = qkv + (row0 + (live ? t : 0)) * ld + h * kHD;
#pragma unroll
    for (int i = 0; i < kHD; i += 4) {
      const float4 v = *(const float4*)(qp + i);
      q[i] = v.x * scale; q[i + 1] = v.y * scale; q[i + 2] = v.z * scale; q[i + 3] = v.w * scale;
    }
  }
#pragma unroll
  for (int i = 0; i < kHD; ++i) o[i] = 0.f;
  float mx = -INFINITY, l = 0.f;
  const int k_lo = max(0, t0 - window + 1), k_hi = min(S - 1, t0 + kQT - 1);
  for (int c0 = k_lo; c0 <= k_hi; c0 += kKC) {
    __syncthreads();
    for (int i = lane; i < kKC * (kHD / 4); i += 64) {
      const int j = i / (kHD / 4), d4 = i - j * (kHD / 4);
      const int key = min(c0 + j, S - 1);
      const float* kp = qkv + (row0 + key) * ld + kD + h * kHD + 4 * d4;
      ks[j][d4] = *(const float4*)kp;
      vs[j][d4] = *(const float4*)(kp + kD);
    }
    __syncthreads();
    float sc[kKC];
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKC; ++j) {
      const int key = c0 + j;
      const bool ok = live && key <= k_hi && key <= t && key > t - window;
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < kHD / 4; ++i) {
        const float4 kv = ks[j][i];
        d = fmaf(q[4 * i], kv.x, d);
        d = fmaf(q[4 * i + 1], kv.y, d);
        d = fmaf(q[4 * i + 2], kv.z, d);
        d = fmaf(q[4 * i + 3], kv.w, d);
      }
      sc[j] = ok ? d : -INFINITY;
      cm = fmaxf(cm, sc[j]);
    }
    const float nm = fmaxf(mx, cm);
    if (nm == -INFINITY) continue;  // nothing allowed yet for this query
    const float corr = expf(mx - nm);  // exp(-inf) = 0 on the first allowed chunk
    l *= corr;
#pragma unroll
    for (int i = 0; i < kHD; ++i) o[i] *= corr;
    mx = nm;
#pragma unroll
    for (int j = 0; j < kKC; ++j) {
      const float p = expf(sc[j] - nm);
      l += p;
#pragma unroll
      for (int i = 0; i < kHD / 4; ++i) {
        const float4 vv = vs[j][i];
        o[4 * i] = fmaf(p, vv.x, o[4 * i]);
        o[4 * i + 1] = fmaf(p, vv.y, o[4 * i + 1]);
        o[4 * i + 2] = fmaf(p, vv.z, o[4 * i + 2]);
        o[4 * i + 3] = fmaf(p, vv.w, o[4 * i + 3]);
      }
    }
  }
  if (!live) return;
  const float inv = 1.f / l;
  float* op = out + (row0 + t) * kD + h * kHD;
#pragma unroll
  for (int i = 0; i < kHD; i += 4)
    *(float4*)(op + i) = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
}

// floats of one layer's packed weights, in the order ln1 g/b, Wq, Wk, Wv, Wo,
// scale1, ln2 g/b, W1, W2, scale2
constexpr long long kLayerFloats = 2LL * kD + 4LL * kD * kD + kD + 2LL * kD + 2LL * kF * kD + kD;

}  // namespace

extern "C" {

size_t moshi_mimi_transformer_work_bytes(int32_t B, int32_t S) {
  if (B < 0 || S < 0) return 0;
  const size_t M = (size_t)B * S;
  return (M * (kD + 3 * kD + kD + kF) + (size_t)S * kHD) * sizeof(float);
}

int moshi_mimi_transformer(float* x, int32_t B, int32_t S, const float* weights, int32_t n_layers, int32_t window,
                           void* work, void* hip_stream) {
  if (B < 0 || S < 0 || n_layers < 0 || n_layers > 64 || window < 1) return MOSHI_EINVAL;
  if ((long long)B * S == 0 || n_layers == 0) return MOSHI_OK;
  if (!x || !weights || !work) return MOSHI_EINVAL;
  if ((long long)B * S > (1LL << 24)) return MOSHI_EINVAL;
  hipStream_t s = (hipStream_t)hip_stream;
  const int M = B * S;
  float* nb = (float*)work;
  float* qkv = nb + (size_t)M * kD;
  float* att = qkv + (size_t)M * 3 * kD;
  float* mlp = att + (size_t)M * kD;
  float* rope = mlp + (size_t)M * kF;
  k_rope_table64<<<(unsigned)((S * (kHD / 2) + 255) / 256), 256, 0, s>>>(rope, S, kHD);
  const unsigned ln_blocks = (unsigned)((M + 3) / 4);
  for (int l = 0; l < n_layers; ++l) {
    const float* w = weights + (size_t)l * kLayerFloats;
    const float *ln1g = w, *ln1b = w + kD, *wqkv = w + 2 * kD, *wo = wqkv + 3LL * kD * kD, *sc1 = wo + (long long)kD * kD;
    const float *ln2g = sc1 + kD, *ln2b = ln2g + kD, *w1 = ln2b + kD, *w2 = w1 + (long long)kF * kD;
    const float* sc2 = w2 + (long long)kD * kF;
    k_layer_norm<<<ln_blocks, 256, 0, s>>>(x, ln1g, ln1b, nb, M);
    GemmAux ra;
    ra.rope = rope;
    ra.rope_cols = 2 * kD;
    ra.hd = kHD;
    ra.seq = S;
    gemm_f32<G_ROPE>(nb, wqkv, qkv, M, 3 * kD, kD, ra, s);
    k_window_attn<<<dim3((S + kQT - 1) / kQT, kH, B), 64, 0, s>>>(qkv, att, S, window);
    GemmAux r1;
    r1.scale = sc1;
    gemm_f32<G_SCALE_RESID>(att, wo, x, M, kD, kD, r1, s);
    k_layer_norm<<<ln_blocks, 256, 0, s>>>(x, ln2g, ln2b, nb, M);
    gemm_f32<G_GELU>(nb, w1, mlp, M, kF, kD, GemmAux{}, s);
    GemmAux r2;
    r2.scale = sc2;
    gemm_f32<G_SCALE_RESID>(mlp, w2, x, M, kD, kF, r2, s);
  }
  return hipGetLastError() == hipSuccess ? MOSHI_OK : MOSHI_EHIP;
}

}  // extern "C"
