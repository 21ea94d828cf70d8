// Tiled float32 GEMM Y[M][N] = X[M][K] W[N][K]^T on the vector units, with
// fused epilogues, for the codec-side maps (Mimi's quantiser projections and
// bottleneck Transformer). 64 x 64 output tile per 256-thread block, 4 x 4
// outputs per thread, K staged through LDS 16 columns at a time; a thread's 4
// output columns are consecutive, so RoPE pairs stay in one thread.
// Requirements (checked by the callers): N % 64 == 0, K % 16 == 0, rows of X
// and W 16-byte aligned.
#pragma once
#include <hip/hip_runtime.h>

namespace moshi_f32 {

enum GemmEpi {
  G_STORE = 0,       // Y = acc
  G_ROPE = 1,        // Y = acc, columns < rope_cols rotated by position (row % seq) (table [seq][hd/2][2])
  G_GELU = 2,        // Y = GELU(acc) (erf form)
  G_SCALE_RESID = 3  // Y += scale[n] * acc
};

struct GemmAux {
  const float* scale = nullptr;  // G_SCALE_RESID: [N]
  const float* rope = nullptr;   // G_ROPE: [seq][hd/2] (cos, sin)
  int rope_cols = 0, hd = 0, seq = 1;
};

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* X, const float* W, float* Y, int M, int N, int K,
                                                  GemmAux aux, int rows_on_x) {
  __shared__ float4 As[16][16 + 1];  // [k][64 rows as 16 float4]
  __shared__ float4 Bs[16][16 + 1];
  const int tid = threadIdx.x;
  // column tiles on x (consecutive blocks share the input rows), unless there are
  // more row tiles than grid y holds
  const int m0 = (rows_on_x ? blockIdx.x : blockIdx.y) * 64, n0 = (rows_on_x ? blockIdx.y : blockIdx.x) * 64;
  const int ti = tid / 16, tj = tid % 16;  // rows 4ti.., cols 4tj..
  float acc[4][4] = {};
  const int lr = tid / 4, lk = (tid % 4) * 4;  // loader: row lr, columns lk..lk+3
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 xa = (m0 + lr < M) ? *(const float4*)(X + (long long)(m0 + lr) * K + k0 + lk)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 wb = *(const float4*)(W + (long long)(n0 + lr) * K + k0 + lk);
    __syncthreads();
    ((float*)&As[lk + 0][lr / 4])[lr % 4] = xa.x;
    ((float*)&As[lk + 1][lr / 4])[lr % 4] = xa.y;
    ((float*)&As[lk + 2][lr / 4])[lr % 4] = xa.z;
    ((float*)&As[lk + 3][lr / 4])[lr % 4] = xa.w;
    ((float*)&Bs[lk + 0][lr / 4])[lr % 4] = wb.x;
    ((float*)&Bs[lk + 1][lr / 4])[lr % 4] = wb.y;
    ((float*)&Bs[lk + 2][lr / 4])[lr % 4] = wb.z;
    ((float*)&Bs[lk + 3][lr / 4])[lr % 4] = wb.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float4 a = As[k][ti], b = Bs[k][tj];
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
  }
  const int n = n0 + tj * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ti * 4 + i;
    if (m >= M) continue;
    float* y = Y + (long long)m * N + n;
    float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    if constexpr (EPI == G_ROPE) {
      if (n < aux.rope_cols) {
        const int pos = m % aux.seq;
        const int dim = n % aux.hd;  // even
#pragma unroll
        for (int p = 0; p < 4; p += 2) {
          const float* cs = aux.rope + ((long long)pos * (aux.hd / 2) + (dim + p) / 2) * 2;
          const float x0 = v[p], x1 = v[p + 1];
          v[p] = x0 * cs[0] - x1 * cs[1];
          v[p + 1] = x0 * cs[1] + x1 * cs[0];
        }
      }
    }
    if constexpr (EPI == G_GELU) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = 0.5f * v[j] * (1.f + erff(v[j] * 0.70710678118654752f));
    }
    if constexpr (EPI == G_SCALE_RESID) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = fmaf(aux.scale[n + j], v[j], y[j]);
    }
    *(float4*)y = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int EPI>
inline void gemm_f32(const float* X, const float* W, float* Y, int M, int N, int K, const GemmAux& aux,
                     hipStream_t s) {
  const int mt = (M + 63) / 64, nt = N / 64;
  const int rows_on_x = mt > 65535 ? 1 : 0;
  const dim3 grid(rows_on_x ? mt : nt, rows_on_x ? nt : mt);
  k_gemm_f32<EPI><<<grid, 256, 0, s>>>(X, W, Y, M, N, K, aux, rows_on_x);
}

}  // namespace moshi_f32
