// Cross-entropy of teacher-forced scoring (Moshi walkthrough on 139.9.1.231,
// section "训练损失"; loss weights from the notes page "Moshi: a Speech-Text
// Foundation Model for Real-Time Dialogue", section 4): per-position values
// first, then one deterministic reduction.
#include <hip/hip_runtime.h>

#include <math.h>

#include "moshi_internal.h"

namespace moshi {

// ce[(b * S + s) * 9 + slot] = logsumexp(l) - l[target], or -1 for a pad target.
__global__ __launch_bounds__(256) void k_ce_rows(CeRowsArgs a) {
  const int b = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const int n = slot == 0 ? a.vocab_text : a.codebook;
  const float* l = slot == 0 ? a.text_logits + (long long)b * a.ld_text
                             : a.audio_logits + (long long)b * a.ld_audio + (long long)(slot - 1) * a.codebook;
  const int t = a.targets[b * a.tgt_stride + slot];
  const int pad = slot == 0 ? a.vocab_text : a.codebook;
  double* out = a.ce + ((long long)b * a.S + a.s) * kSlots + slot;
  if (t == pad || t < 0 || t > pad) {
    if (tid == 0) *out = -1.0;
    return;
  }
  __shared__ float s_f[256];
  __shared__ double s_d[256];
  float m = -INFINITY;
  for (int i = tid; i < n; i += 256) m = fmaxf(m, l[i]);
  s_f[tid] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_f[tid] = fmaxf(s_f[tid], s_f[tid + o]);
    __syncthreads();
  }
  m = s_f[0];
  double sum = 0.0;
  for (int i = tid; i < n; i += 256) sum += (double)expf(l[i] - m);
  s_d[tid] = sum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_d[tid] += s_d[tid + o];
    __syncthreads();
  }
  if (tid == 0) *out = log(s_d[0]) + (double)m - (double)l[t];
}

void launch_ce_rows(const CeRowsArgs& a, int B, bool with_audio, hipStream_t s) {
  dim3 grid(B, with_audio ? kSlots : 1);
  k_ce_rows<<<grid, 256, 0, s>>>(a);
}

// res[0..8]: mean CE per slot over non-pad targets; res[9..17]: counts;
// res[18] = ce_audio = sum_j alpha_j CE_j / sum_j alpha_j (alpha = 100, 1, ..., 1);
// res[19] = ce_text + ce_audio.
__global__ __launch_bounds__(256) void k_ce_reduce(const double* ce, long long n_rows, int n_slots, double* res) {
  __shared__ double s_sum[256];
  __shared__ double s_cnt[256];
  const int tid = threadIdx.x;
  for (int slot = 0; slot < kSlots; ++slot) {
    double sum = 0.0, cnt = 0.0;
    if (slot < n_slots) {
      for (long long i = tid; i < n_rows; i += 256) {
        const double v = ce[i * kSlots + slot];
        if (v >= 0.0) {
          sum += v;
          cnt += 1.0;
        }
      }
    }
    s_sum[tid] = sum;
    s_cnt[tid] = cnt;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        s_sum[tid] += s_sum[tid + o];
        s_cnt[tid] += s_cnt[tid + o];
      }
      __syncthreads();
    }
    if (tid == 0) {
      res[slot] = s_cnt[0] > 0 ? s_sum[0] / s_cnt[0] : 0.0;
      res[kSlots + slot] = s_cnt[0];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double num = 0.0, den = 0.0;
    for (int j = 0; j < 8; ++j) {
      const double alpha = j == 0 ? 100.0 : 1.0;
      num += alpha * res[1 + j];
      den += alpha;
    }
    res[18] = n_slots > 1 ? num / den : 0.0;
    res[19] = res[0] + res[18];
  }
}

void launch_ce_reduce(const double* ce, long long n_rows, int n_slots, double* res, hipStream_t s) {
  k_ce_reduce<<<1, 256, 0, s>>>(ce, n_rows, n_slots, res);
}

// RoPE angles in double precision: out[p][i] = (cos, sin)(p * base^(-2i/hd)).
__global__ void k_rope_table(float* out, int P, int hd, double base) {
  const int half = hd / 2;
  const long long total = (long long)P * half;
  for (long long t = blockIdx.x * 256LL + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
    const int p = (int)(t / half), i = (int)(t - (long long)p * half);
    const double ang = (double)p * pow(base, -2.0 * i / hd);
    out[t * 2] = (float)cos(ang);
    out[t * 2 + 1] = (float)sin(ang);
  }
}

void launch_rope_table(float* out, int P, int hd, double base, hipStream_t s) {
  long long total = (long long)P * (hd / 2);
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  k_rope_table<<<blocks, 256, 0, s>>>(out, P, hd, base);
}

}  // namespace moshi
