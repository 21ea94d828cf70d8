// Split residual vector quantiser of the Mimi codec (walkthrough of the Moshi
// report, sections "量化率" and "使用分裂RVQ学习语义-声学token", Fig. 2; notes
// page section 3a): a 512 -> 256 input projection, a plain VQ (semantic
// codebook 0) and a 7-level RVQ (acoustic codebooks 1..7) applied in parallel
// to the projected latent, their codewords summed and projected back to 512.
//
// Kernels: the tiled float32 GEMM of gemm_f32.h for the two projections, codeword norms, and one
// nearest-codeword kernel per level. A block owns 32 latent rows (in LDS) and
// walks the codebook in chunks of 32 codewords staged in LDS as 16-byte groups
// of 4 dimensions per codeword; lane l of a wave scores codeword l % 32 against
// 4 of the wave's 8 rows (row groups read as broadcasts) with
// distance ||c||^2 - 2 r.c (||r||^2 is common to a row), keeping the lowest
// index on ties. An acoustic level then subtracts the chosen codewords from its
// rows and writes the residual back.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/moshi.h"
#include "gemm_f32.h"

namespace {

constexpr int kRows = 32;   // latent rows per block (4 waves x 8)
constexpr int kChunk = 32;  // codewords per LDS chunk
constexpr int kMaxDim = 256;

// ||c||^2 of every codeword, summed in dimension order
__global__ void k_code_norms(const float* C, float* norms, long long n, int D) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float* c = C + i * D;
  float s = 0.f;
  for (int k = 0; k < D; ++k) s = fmaf(c[k], c[k], s);
  norms[i] = s;
}

__device__ __forceinline__ void keep_lower(float& bd, int& bi, float d, int i) {
  if (d < bd || (d == bd && i < bi)) {
    bd = d;
    bi = i;
  }
}

// One quantiser level over rows [blockIdx.x * 32, +32) of `in` [M][D]: codes of
// level q into codes[m * Q + q]; with `out` set, out = in - C[code] (the
// acoustic residual; in and out may alias, a block owns its rows).
__global__ __launch_bounds__(256) void k_rvq_level(const float* in, float* out, const float* C, const float* norms,
                                                   int N, int D, int M, int* codes, int Q, int q) {
  __shared__ float4 rows4[kRows][kMaxDim / 4];
  __shared__ float4 cs4[kMaxDim / 4][kChunk];  // [4 dims][codeword]: one 16-byte read per lane
  __shared__ int best_idx[kRows];
  float* rows = (float*)rows4;  // [kRows][kMaxDim]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * kRows;
  const int D4 = D / 4;
  for (int i = tid; i < kRows * D4; i += 256) {
    const int r = i / D4, k4 = i - r * D4;
    rows4[r][k4] = (m0 + r < M) ? *(const float4*)(in + (long long)(m0 + r) * D + 4 * k4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // lane: codeword lane % 32 of a chunk, rows wave*8 + (lane / 32) * 4 + 0..3
  const int cl = lane & 31, r0 = wave * 8 + (lane >> 5) * 4;
  float bd[4];
  int bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bd[i] = INFINITY;
    bi[i] = 0x7fffffff;
  }
  for (int c0 = 0; c0 < N; c0 += kChunk) {
    __syncthreads();  // the previous chunk is consumed (and, first time, rows are in)
    for (int i = tid; i < kChunk * D4; i += 256) {
      const int c = i / D4, k4 = i - c * D4;
      cs4[k4][c] = (c0 + c < N) ? *(const float4*)(C + (long long)(c0 + c) * D + 4 * k4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    float dot[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k4 = 0; k4 < D4; ++k4) {
      const float4 cv = cs4[k4][cl];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 rv = rows4[r0 + i][k4];
        dot[i] = fmaf(rv.x, cv.x, dot[i]);
        dot[i] = fmaf(rv.y, cv.y, dot[i]);
        dot[i] = fmaf(rv.z, cv.z, dot[i]);
        dot[i] = fmaf(rv.w, cv.w, dot[i]);
      }
    }
    const int c = c0 + cl;
    if (c < N) {
      const float nc = norms[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) keep_lower(bd[i], bi[i], fmaf(-2.f, dot[i], nc), c);
    }
  }
  // argmin over the 32 lanes sharing a row set
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      const float od = __shfl_xor(bd[i], o, 64);
      const int oi = __shfl_xor(bi[i], o, 64);
      keep_lower(bd[i], bi[i], od, oi);
    }
  }
  if (cl == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) best_idx[r0 + i] = bi[i];
  }
  __syncthreads();
  if (tid < kRows && m0 + tid < M) codes[(long long)(m0 + tid) * Q + q] = best_idx[tid] < N ? best_idx[tid] : 0;
  if (!out) return;
  for (int i = tid; i < kRows * D; i += 256) {
    const int r = i / D, k = i - r * D;
    const int b = best_idx[r] < N ? best_idx[r] : 0;  // NaN distances keep no index
    if (m0 + r < M) out[(long long)(m0 + r) * D + k] = rows[r * kMaxDim + k] - C[(long long)b * D + k];
  }
}

// y[m][k] = sum over levels of C_q[codes[m][q]][k]
__global__ void k_rvq_sum(const int* codes, const float* C, int Q, int N, int D, int M, float* y) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i >= (long long)M * D) return;
  const long long m = i / D;
  const int k = (int)(i - m * D);
  float s = 0.f;
  for (int q = 0; q < Q; ++q) {
    int c = codes[m * Q + q];
    c = c < 0 ? 0 : (c >= N ? N - 1 : c);
    s += C[((long long)q * N + c) * D + k];
  }
  y[i] = s;
}

void linear(const float* X, const float* W, float* Y, int M, int N, int K, hipStream_t s) {
  moshi_f32::gemm_f32<moshi_f32::G_STORE>(X, W, Y, M, N, K, moshi_f32::GemmAux{}, s);
}

bool bad_shape(int32_t M, int32_t dz, int32_t dq, int32_t Q, int32_t N) {
  return M < 0 || dz < 64 || dz % 64 || dq < 64 || dq % 64 || dq > kMaxDim || Q < 2 || Q > 32 || N < 1 ||
         N > (1 << 20);
}

}  // namespace

extern "C" {

size_t moshi_rvq_work_bytes(int32_t M, int32_t dq, int32_t Q, int32_t N) {
  if (M < 0 || dq < 1 || Q < 1 || N < 1) return 0;
  return ((size_t)2 * M * dq + (size_t)Q * N) * sizeof(float);
}

int moshi_rvq_encode(const float* z, int32_t M, int32_t dz, const float* w_in, int32_t dq, const float* codebooks,
                     int32_t Q, int32_t N, int32_t* codes, void* work, void* hip_stream) {
  if (bad_shape(M, dz, dq, Q, N)) return MOSHI_EINVAL;
  if (M == 0) return MOSHI_OK;
  if (!z || !w_in || !codebooks || !codes || !work) return MOSHI_EINVAL;
  hipStream_t s = (hipStream_t)hip_stream;
  float* X = (float*)work;
  float* R = X + (size_t)M * dq;
  float* norms = R + (size_t)M * dq;
  const long long nq = (long long)Q * N;
  k_code_norms<<<(unsigned)((nq + 255) / 256), 256, 0, s>>>(codebooks, norms, nq, dq);
  linear(z, w_in, X, M, dq, dz, s);
  const unsigned blocks = (unsigned)((M + kRows - 1) / kRows);
  // semantic VQ on the projected latent; acoustic RVQ from the same latent
  k_rvq_level<<<blocks, 256, 0, s>>>(X, nullptr, codebooks, norms, N, dq, M, codes, Q, 0);
  for (int q = 1; q < Q; ++q)
    k_rvq_level<<<blocks, 256, 0, s>>>(q == 1 ? X : R, R, codebooks + (size_t)q * N * dq, norms + (size_t)q * N, N,
                                       dq, M, codes, Q, q);
  return hipGetLastError() == hipSuccess ? MOSHI_OK : MOSHI_EHIP;
}

int moshi_rvq_decode(const int32_t* codes, int32_t M, const float* codebooks, int32_t Q, int32_t N, int32_t dq,
                     const float* w_out, int32_t dz, float* z_hat, void* work, void* hip_stream) {
  if (bad_shape(M, dz, dq, Q, N)) return MOSHI_EINVAL;
  if (M == 0) return MOSHI_OK;
  if (!codes || !codebooks || !w_out || !z_hat || !work) return MOSHI_EINVAL;
  hipStream_t s = (hipStream_t)hip_stream;
  float* Y = (float*)work;
  const long long n = (long long)M * dq;
  k_rvq_sum<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(codes, codebooks, Q, N, dq, M, Y);
  linear(Y, w_out, z_hat, M, dz, dq, s);
  return hipGetLastError() == hipSuccess ? MOSHI_OK : MOSHI_EHIP;
}

}  // extern "C"
