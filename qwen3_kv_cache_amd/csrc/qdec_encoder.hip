// Audio frontend and SAN-M encoder kernels (the GEMMs and the attention are
// the prefill kernels of qdec_kernels.hip).
//
// Frontend (audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan",
// Task 2 Step 4; transcribe.cpp "Forward map - funasr_nano", table
// "Frontend"): one workgroup per 25 ms frame computes, in float64, the
// frame's mean removal, 0.97 pre-emphasis, Hamming window, a 512-point FFT
// in LDS (radix 2), the power of bins 0 .. 255, 80 HTK-mel triangle energies
// and their natural log (floor: the float32 epsilon). The work is a few
// microseconds of ALU per frame; float64 keeps the far-from-peak mel energies
// of tonal inputs (1e-8 of the peak) accurate to far below the log tolerance.
//
// Encoder glue (same plan, Tasks 3-4; the map's "Encoder" table): LFR
// stacking with the sqrt(dim) scale and the sinusoidal positions, the FSMN
// memory v + depthwise conv(v) over time added into the residual stream, and
// LayerNorm into fp32.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "qdec_internal.h"

namespace qdec {
namespace {

constexpr int kFftN = 512;
constexpr int kFftHalf = kFftN / 2;

__device__ double block_sum_d(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < (int)(blockDim.x / 64); ++i) s += red[i];
  return s;
}

// grid: one workgroup (256 threads) per frame
__global__ __launch_bounds__(256) void fbank_kernel(const float* __restrict__ pcm, FrontTables tb,
                                                    float* __restrict__ out) {
  __shared__ double re[kFftN];
  __shared__ double im[kFftN];
  __shared__ double a[kFrameLen];
  __shared__ double red[4];
  const int f = blockIdx.x, tid = threadIdx.x;
  const float* x = pcm + (size_t)f * kFrameShift;
  double s = 0.0;
  for (int i = tid; i < kFrameLen; i += 256) {
    a[i] = (double)x[i];
    s += a[i];
  }
  const double mean = block_sum_d(s, red) / kFrameLen;
  for (int i = tid; i < kFrameLen; i += 256) a[i] -= mean;
  __syncthreads();
  // pre-emphasis (sample 0 against itself), window, zero padding; stored at
  // the bit-reversed index for the in-place FFT
  for (int i = tid; i < kFftN; i += 256) {
    double y = 0.0;
    if (i < kFrameLen) y = (a[i] - kPreemph * a[i > 0 ? i - 1 : 0]) * tb.window[i];
    const int r = __brev((unsigned)i) >> (32 - 9);
    re[r] = y;
    im[r] = 0.0;
  }
  __syncthreads();
  // radix-2 stages: butterfly `tid` of the stage with half-size h uses the
  // twiddle exp(-2 pi i j / (2 h)) = tw[j * (kFftHalf / h)]
  for (int h = 1; h < kFftN; h <<= 1) {
    const int j = tid & (h - 1);
    const int i0 = ((tid - j) << 1) + j, i1 = i0 + h;
    const int k = j * (kFftHalf / h);
    const double wr = tb.tw_re[k], wi = tb.tw_im[k];
    const double br = re[i1] * wr - im[i1] * wi, bi = re[i1] * wi + im[i1] * wr;
    const double ar = re[i0], ai = im[i0];
    re[i0] = ar + br;
    im[i0] = ai + bi;
    re[i1] = ar - br;
    im[i1] = ai - bi;
    __syncthreads();
  }
  // power of bins 0 .. 255 (thread k), into re
  const double p = re[tid] * re[tid] + im[tid] * im[tid];
  __syncthreads();
  re[tid] = p;
  __syncthreads();
  if (tid < kMels) {
    const int lo = tb.mel_lo[tid], hi = tb.mel_hi[tid];
    const double* w = tb.mel_w + (size_t)tid * kFftHalf;
    double e = 0.0;
    for (int b = lo; b < hi; ++b) e += w[b] * re[b];
    out[(size_t)f * kMels + tid] = (float)log(fmax(e, (double)FLT_EPSILON));
  }
}

// grid: one workgroup per LFR row t. Row t stacks frames
// clamp(t n + j - (m - 1) / 2, 0, T - 1), j = 0 .. m - 1. lfr (optional)
// receives the stacked row, x0 (optional) the row times `scale` plus the
// sinusoid PE[t, 2i] = sin(t w_i), PE[t, 2i + 1] = cos(t w_i).
__global__ __launch_bounds__(256) void lfr_embed_kernel(const float* __restrict__ fb, int T, int n_mels, int m,
                                                        int n, float scale, const double* __restrict__ inv_freq,
                                                        float* __restrict__ lfr, float* __restrict__ x0) {
  const int t = blockIdx.x, W = n_mels * m, left = (m - 1) / 2;
  for (int c = threadIdx.x; c < W; c += 256) {
    const int j = c / n_mels, mel = c - j * n_mels;
    const int src = min(max(t * n + j - left, 0), T - 1);
    const float v = fb[(size_t)src * n_mels + mel];
    if (lfr) lfr[(size_t)t * W + c] = v;
    if (x0) {
      const double ang = (double)t * inv_freq[c >> 1];
      const double pe = (c & 1) ? cos(ang) : sin(ang);
      x0[(size_t)t * W + c] = (float)((double)v * (double)scale + pe);
    }
  }
}

// out[t, c] = (accumulate ? out[t, c] : 0) + v[t, c] + sum_j w[c, j] v[t + j - (K-1)/2, c]
// with v = qkv[t, 2 dim + c] (row pitch ld) and zero outside [0, T).
// grid: (dim / 256 rounded up, T)
__global__ __launch_bounds__(256) void fsmn_kernel(const float* __restrict__ qkv, int ld, int T, int dim, int K,
                                                   const float* __restrict__ w, int accumulate,
                                                   float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x, t = blockIdx.y;
  if (c >= dim) return;
  const float* v = qkv + 2 * dim + c;
  const int half = (K - 1) / 2;
  float m = v[(size_t)t * ld];
  for (int j = 0; j < K; ++j) {
    const int u = t + j - half;
    if (u >= 0 && u < T) m = fmaf(w[(size_t)c * K + j], v[(size_t)u * ld], m);
  }
  float* o = out + (size_t)t * dim + c;
  *o = accumulate ? *o + m : m;
}

__device__ float block_sum_f(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x / 64); ++i) s += red[i];
  return s;
}

// LayerNorm (population variance, gain and bias) of row blockIdx.x into fp32;
// out may alias X (every read of the row precedes the first write)
__global__ __launch_bounds__(256) void ln_apply_kernel(const float* X, int K, const float* __restrict__ gain,
                                                       const float* __restrict__ bias, float eps, float* out) {
  __shared__ float red[4];
  const float* x = X + (size_t)blockIdx.x * K;
  float s = 0.f;
  for (int i = threadIdx.x; i < K; i += 256) s += x[i];
  const float mean = block_sum_f(s, red) / (float)K;
  float ss = 0.f;
  for (int i = threadIdx.x; i < K; i += 256) {
    const float c = x[i] - mean;
    ss = fmaf(c, c, ss);
  }
  const float inv = 1.f / sqrtf(block_sum_f(ss, red) / (float)K + eps);
  float* o = out + (size_t)blockIdx.x * K;
  for (int i = threadIdx.x; i < K; i += 256) o[i] = (x[i] - mean) * inv * gain[i] + bias[i];
}

}  // namespace

hipError_t launch_fbank(const float* pcm, int n_frames, const FrontTables& tb, float* out, hipStream_t st) {
  if (n_frames < 1) return hipErrorInvalidValue;
  fbank_kernel<<<n_frames, 256, 0, st>>>(pcm, tb, out);
  return hipGetLastError();
}

hipError_t launch_lfr_embed(const float* fb, int T, int n_mels, int m, int n, float scale, const double* inv_freq,
                            float* lfr, float* x0, int rows, hipStream_t st) {
  if (rows < 1 || T < 1 || n_mels * m > 65536) return hipErrorInvalidValue;
  lfr_embed_kernel<<<rows, 256, 0, st>>>(fb, T, n_mels, m, n, scale, inv_freq, lfr, x0);
  return hipGetLastError();
}

hipError_t launch_fsmn(const float* qkv, int ld, int T, int dim, int K, const float* w, bool accumulate, float* out,
                       hipStream_t st) {
  if (T < 1 || dim < 1 || K < 1 || (K & 1) == 0 || ld < 3 * dim) return hipErrorInvalidValue;
  fsmn_kernel<<<dim3((dim + 255) / 256, T), 256, 0, st>>>(qkv, ld, T, dim, K, w, accumulate ? 1 : 0, out);
  return hipGetLastError();
}

hipError_t launch_ln_apply(const float* X, int T, int K, const float* gain, const float* bias, float eps, float* out,
                           hipStream_t st) {
  ln_apply_kernel<<<T, 256, 0, st>>>(X, K, gain, bias, eps, out);
  return hipGetLastError();
}

}  // namespace qdec
