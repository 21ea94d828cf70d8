// SEANet causal convolutional encoder and decoder of the Mimi codec (walkthrough
// of the Moshi report, section on Mimi's baseline architecture; notes page
// section 3a): a mono 24 kHz waveform <-> 512-dim latents at 12.5 frames/s.
//
// Layout per stage: channel-major [B][C][T] float32. Encoder: kernel-7 input
// convolution to 64 channels; per stride (4, 5, 6, 8) a residual unit
// x + conv_k1(ELU(conv_k3(ELU(x)))) and an ELU + strided convolution (kernel
// 2 * stride) doubling the channels; an ELU + kernel-4 stride-2 convolution to
// 512, written frame-major [B][S][512]. Decoder: kernel-4 stride-2 transposed
// convolution from [B][S][512] to 1024 channels, then per stride (8, 6, 5, 4)
// an ELU + transposed convolution halving the channels and a residual unit;
// an ELU + kernel-7 convolution to one channel. Causal padding: (k-1)*d + 1 - s
// zeros on the left; transposed outputs past T_in * s are dropped. No biases.
//
// Every convolution writes its raw output and/or the ELU of it (whichever its
// consumers read), so no kernel recomputes ELU on its inputs; the residual
// unit's skip is added in the second convolution's epilogue. An LDS-tiled
// implicit-GEMM kernel runs the convolutions (a direct kernel the one-channel
// ends); a transposed convolution runs as its stride's phases, each a causal
// 2-tap convolution writing every s-th sample.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/moshi.h"

namespace {

constexpr int kFrame = 1920;  // samples per latent frame (4 * 5 * 6 * 8 * 2)
constexpr int kBase = 64, kDim = 512;
constexpr int kStrides[4] = {4, 5, 6, 8};
struct ConvArgs {
  const float* x;  // [B][Cin][Tin], or [B][Tin][Cin] when in_tc
  const float* w;  // [Cout][Cin][K]
  float* y;        // raw output (channel-major rows of tlen, or [B][tlen][Cout] when out_tc), may be null
  float* ye;       // ELU of the output, channel-major, may be null
  const float* resid;  // added to the output, channel-major, may be null (may equal y)
  int cin, cout, tin, tout, k, stride, pad;
  int ots = 1, oto = 0, tlen = 0;  // output time t goes to t * ots + oto of rows of tlen
  int in_tc = 0, out_tc = 0;
};

constexpr int kTC = 64, kTT = 64;
constexpr int kWsFloats = 8192;  // weights of one input-channel chunk [ci][k][64 co]
constexpr int kXsFloats = 4168;  // input windows of one chunk [ci][63 * s + K]

// input channels per LDS round: as many as the weight and window budgets allow
__host__ __device__ inline int chunk_channels(int K, int stride) {
  const int win = (kTT - 1) * stride + K;
  int ci = kWsFloats / (K * kTC);
  if (kXsFloats / win < ci) ci = kXsFloats / win;
  return ci < 64 ? ci : 64;
}

// Causal convolution as an implicit GEMM: block tile of 64 output channels x 64
// output times, 4 x 4 per thread (channels 4*ti.., times tj + 16*j); a round
// stages CI input channels (chunk_channels): weights [ci][k][co] and the input
// windows [ci][t0*s - pad, + 63*s + K) in LDS.
__global__ __launch_bounds__(256) void k_conv_tiled(ConvArgs a) {
  __shared__ __align__(16) float ws[kWsFloats];
  __shared__ float xs[kXsFloats];
  const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
  const int t0 = blockIdx.x * kTT, co0 = blockIdx.y * kTC, b = blockIdx.z;
  const float* xb = a.x + (long long)b * a.cin * a.tin;
  const int K = a.k, st = a.stride;
  const int win = (kTT - 1) * st + K;
  const int CI = chunk_channels(K, st);
  const int base = t0 * st - a.pad;
  float acc[4][4] = {};
  for (int c0 = 0; c0 < a.cin; c0 += CI) {
    __syncthreads();
    for (int i = tid; i < CI * K * kTC; i += 256) {
      const int co = i % kTC, k = (i / kTC) % K, ci = i / (kTC * K);
      const bool ok = co0 + co < a.cout && c0 + ci < a.cin;
      ws[i] = ok ? a.w[((long long)(co0 + co) * a.cin + c0 + ci) * K + k] : 0.f;
    }
    for (int i = tid; i < CI * win; i += 256) {
      const int ci = i / win, w = i - ci * win;
      const int t = base + w;
      float v = 0.f;
      if (c0 + ci < a.cin && t >= 0 && t < a.tin)
        v = a.in_tc ? xb[(long long)t * a.cin + c0 + ci] : xb[(long long)(c0 + ci) * a.tin + t];
      xs[i] = v;
    }
    __syncthreads();
    const int nci = min(CI, a.cin - c0);
    for (int ci = 0; ci < nci; ++ci) {
      const float* wr = ws + ci * K * kTC + 4 * ti;
      const float* xr = xs + ci * win + tj * st;
      for (int k = 0; k < K; ++k) {
        const float4 wv = *(const float4*)(wr + k * kTC);
        const float av[4] = {wv.x, wv.y, wv.z, wv.w};
        float bv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = xr[16 * j * st + k];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      }
    }
  }
  const int tlen = a.tlen ? a.tlen : a.tout;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int co = co0 + 4 * ti + i;
    if (co >= a.cout) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + tj + 16 * j;
      if (t >= a.tout) continue;
      const long long to = (long long)t * a.ots + a.oto;
      const long long cm = ((long long)b * a.cout + co) * tlen + to;
      float v = acc[i][j];
      if (a.resid) v += a.resid[cm];
      if (a.y) a.y[a.out_tc ? ((long long)b * tlen + to) * a.cout + co : cm] = v;
      if (a.ye) a.ye[cm] = v > 0.f ? v : expm1f(v);
    }
  }
}

// Phase r of a transposed convolution with kernel 2s and stride s is a causal
// 2-tap convolution of the input: y[co][q*s + r] = W[ci][co][r+s] x[ci][q-1] +
// W[ci][co][r] x[ci][q]. Its weights [r][co][ci][2]:
__global__ void k_tconv_phase_weights(const float* w, float* wp, int cin, int cout, int s) {
  const long long i = blockIdx.x * 256LL + threadIdx.x;
  const long long n = (long long)s * cout * cin;
  if (i >= n) return;
  const int ci = (int)(i % cin);
  const int co = (int)((i / cin) % cout);
  const int r = (int)(i / ((long long)cin * cout));
  const long long src = ((long long)ci * cout + co) * (2 * s);
  wp[2 * i] = w[src + r + s];
  wp[2 * i + 1] = w[src + r];
}

// The thin convolutions (one input or one output channel: the waveform ends) run
// one thread per output time over all channels and taps; the weights are uniform
// across the block and consecutive threads read consecutive samples.
__global__ __launch_bounds__(256) void k_conv_direct(ConvArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x, b = blockIdx.z;
  if (t >= a.tout) return;
  const float* xb = a.x + (long long)b * a.cin * a.tin;
  const int base = t * a.stride - a.pad;
  const int tlen = a.tlen ? a.tlen : a.tout;
  for (int co = 0; co < a.cout; ++co) {
    float acc = 0.f;
    for (int ci = 0; ci < a.cin; ++ci) {
      const float* w = a.w + ((long long)co * a.cin + ci) * a.k;
      for (int k = 0; k < a.k; ++k) {
        const int ti = base + k;
        if (ti >= 0 && ti < a.tin) acc = fmaf(w[k], xb[(long long)ci * a.tin + ti], acc);
      }
    }
    const long long to = (long long)t * a.ots + a.oto;
    const long long cm = ((long long)b * a.cout + co) * tlen + to;
    if (a.resid) acc += a.resid[cm];
    if (a.y) a.y[a.out_tc ? ((long long)b * tlen + to) * a.cout + co : cm] = acc;
    if (a.ye) a.ye[cm] = acc > 0.f ? acc : expm1f(acc);
  }
}

void launch_conv(const ConvArgs& a, int B, hipStream_t s) {
  if ((a.cin == 1 || a.cout == 1) && !a.in_tc) {
    k_conv_direct<<<dim3((a.tout + 255) / 256, 1, B), 256, 0, s>>>(a);
    return;
  }
  dim3 grid((a.tout + kTT - 1) / kTT, (a.cout + kTC - 1) / kTC, B);
  k_conv_tiled<<<grid, 256, 0, s>>>(a);
}

ConvArgs conv(const float* x, const float* w, int cin, int cout, int tin, int k, int stride) {
  ConvArgs a{};
  a.x = x;
  a.w = w;
  a.cin = cin;
  a.cout = cout;
  a.tin = tin;
  a.tout = tin / stride;
  a.k = k;
  a.stride = stride;
  a.pad = k - stride;  // (k - 1) * 1 + 1 - stride
  a.ots = 1;
  return a;
}

// transposed convolution (kernel 2s, stride s) from its [Cin][Cout][2s] weights:
// the phase weights go to wp (s * Cout * Cin * 2 floats), then one launch per phase
void launch_tconv(ConvArgs a, const float* w, float* wp, int B, hipStream_t s) {
  const int st = a.stride;
  const long long n = (long long)st * a.cout * a.cin;
  k_tconv_phase_weights<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w, wp, a.cin, a.cout, st);
  a.tlen = a.tin * st;
  a.ots = st;
  a.k = 2;
  a.stride = 1;
  a.pad = 1;
  a.tout = a.tin;
  for (int r = 0; r < st; ++r) {
    a.w = wp + (size_t)r * a.cout * a.cin * 2;
    a.oto = r;
    launch_conv(a, B, s);
  }
}

ConvArgs tconv(const float* x, int cin, int cout, int tin, int stride) {
  ConvArgs a{};
  a.x = x;
  a.cin = cin;
  a.cout = cout;
  a.tin = tin;
  a.stride = stride;
  return a;
}

constexpr long long kPhaseFloats = 2LL * 1024 * 512 * 8;  // largest s * Cout * Cin * 2

// work buffers per sequence: 4 of 64 * T floats (raw/ELU ping-pong pairs), one of
// 32 * T (the residual units' inner activations), T = S * 1920; plus the phase
// weights of one transposed convolution
size_t work_floats(long long B, long long S) {
  return (size_t)B * S * kFrame * (4 * kBase + kBase / 2) + kPhaseFloats;
}

}  // namespace

extern "C" {

size_t moshi_seanet_work_bytes(int32_t B, int32_t S) {
  if (B < 0 || S < 0) return 0;
  return work_floats(B, S) * sizeof(float);
}

int moshi_seanet_encode(const float* audio, int32_t B, int32_t S, const float* w, float* latents, void* work,
                        void* hip_stream) {
  if (B < 0 || S < 0) return MOSHI_EINVAL;
  if ((long long)B * S == 0) return MOSHI_OK;
  if (!audio || !w || !latents || !work) return MOSHI_EINVAL;
  if ((long long)S * kFrame * kBase > (1LL << 31) - 1) return MOSHI_EINVAL;
  hipStream_t s = (hipStream_t)hip_stream;
  const long long T = (long long)S * kFrame, big = (long long)B * kBase * T;
  float* P = (float*)work;
  float* Q = P + big;
  float* P2 = Q + big;
  float* Q2 = P2 + big;
  float* R = Q2 + big;  // [B][C/2][T]
  int c = kBase, t = (int)T;
  ConvArgs a = conv(audio, w, 1, kBase, t, 7, 1);
  a.y = P;
  a.ye = Q;
  launch_conv(a, B, s);
  w += (long long)kBase * 7;
  for (int i = 0; i < 4; ++i) {
    const int st = kStrides[i];
    ConvArgs ra = conv(Q, w, c, c / 2, t, 3, 1);
    ra.ye = R;
    launch_conv(ra, B, s);
    w += (long long)(c / 2) * c * 3;
    ConvArgs rb = conv(R, w, c / 2, c, t, 1, 1);
    rb.y = P;
    rb.resid = P;
    rb.ye = Q;
    launch_conv(rb, B, s);
    w += (long long)c * (c / 2);
    ConvArgs dn = conv(Q, w, c, 2 * c, t, 2 * st, st);
    dn.y = P2;
    dn.ye = Q2;
    launch_conv(dn, B, s);
    w += (long long)2 * c * c * 2 * st;
    c *= 2;
    t /= st;
    float* tp = P;
    P = P2;
    P2 = tp;
    tp = Q;
    Q = Q2;
    Q2 = tp;
  }
  ConvArgs out = conv(Q, w, c, kDim, t, 4, 2);
  out.y = latents;
  out.out_tc = 1;
  launch_conv(out, B, s);
  return hipGetLastError() == hipSuccess ? MOSHI_OK : MOSHI_EHIP;
}

int moshi_seanet_decode(const float* latents, int32_t B, int32_t S, const float* w, float* audio, void* work,
                        void* hip_stream) {
  if (B < 0 || S < 0) return MOSHI_EINVAL;
  if ((long long)B * S == 0) return MOSHI_OK;
  if (!audio || !w || !latents || !work) return MOSHI_EINVAL;
  if ((long long)S * kFrame * kBase > (1LL << 31) - 1) return MOSHI_EINVAL;
  hipStream_t s = (hipStream_t)hip_stream;
  const long long T = (long long)S * kFrame, big = (long long)B * kBase * T;
  float* P = (float*)work;
  float* Q = P + big;
  float* P2 = Q + big;
  float* Q2 = P2 + big;
  float* R = Q2 + big;
  int c = 2 * kDim, t = 2 * S;
  float* WP = R + (long long)B * (kBase / 2) * T;
  ConvArgs in = tconv(latents, kDim, c, S, 2);
  in.in_tc = 1;
  in.ye = Q;
  launch_tconv(in, w, WP, B, s);
  w += (long long)kDim * c * 4;
  for (int i = 0; i < 4; ++i) {
    const int st = kStrides[3 - i];
    ConvArgs up = tconv(Q, c, c / 2, t, st);
    up.y = P2;
    up.ye = Q2;
    launch_tconv(up, w, WP, B, s);
    w += (long long)c * (c / 2) * 2 * st;
    c /= 2;
    t *= st;
    ConvArgs ra = conv(Q2, w, c, c / 2, t, 3, 1);
    ra.ye = R;
    launch_conv(ra, B, s);
    w += (long long)(c / 2) * c * 3;
    ConvArgs rb = conv(R, w, c / 2, c, t, 1, 1);
    rb.y = P2;
    rb.resid = P2;
    rb.ye = Q2;
    launch_conv(rb, B, s);
    w += (long long)c * (c / 2);
    float* tp = P;
    P = P2;
    P2 = tp;
    tp = Q;
    Q = Q2;
    Q2 = tp;
  }
  ConvArgs out = conv(Q, w, c, 1, t, 7, 1);
  out.y = audio;
  launch_conv(out, B, s);
  return hipGetLastError() == hipSuccess ? MOSHI_OK : MOSHI_EHIP;
}

}  // extern "C"
