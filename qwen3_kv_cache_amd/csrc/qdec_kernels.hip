// HIP kernels for the Qwen3 KV-cache decoder on gfx950 (CDNA4, wave64):
// prefill and batched decode run layer by layer through these kernels; the
// single-state decode step is the persistent kernel of qdec_decode.hip.
//
// Step map (transcribe.cpp "Forward map - funasr_nano", table "LLM decoder";
// NCNN "Qwen3ASR ncnn多平台移植", section 5):
//   embed + audio-row override   -> embed_prefill_kernel / embed_rows_kernel
//   rms_norm + Q/K/V projection  -> rms_split + gemm
//   per-head Q/K-RMSNorm + NeoX RoPE + KV append -> qk_rope_append_kernel (prefill),
//                                   the prologue of attn_rows_kernel (batched decode)
//   causal GQA attention         -> attn_rows_kernel (batched decode),
//                                   attn_prefill_mfma_kernel / attn_prefill_kernel
//   O projection + residual      -> gemm with the residual epilogue
//   rms_norm + gate_up + SiLU*up -> gemm with the SwiGLU epilogue
//   down projection + residual   -> gemm with the residual epilogue
//   final rms_norm + tied head + greedy argmax -> lm_head_kernel (one row) or gemm +
//                                   argmax_rows_kernel (batch), then argmax_final_kernel
#include <hip/hip_runtime.h>

#include <mutex>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <type_traits>

#include "qdec_internal.h"

namespace qdec {
namespace {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// KV pages as global-address-space pointers. A pointer made from a page-table
// entry is otherwise generic, and generic (flat) accesses count against the
// LDS wait counter as well: every LDS read or cross-lane shuffle after them
// would then also wait for the page loads and stores still in flight.
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) f32x4_t gf32x4;
__device__ __forceinline__ gfloat* page_at(const int64_t* table, int i) { return (gfloat*)table[i]; }
__device__ __forceinline__ float4 gload4(const gfloat* p) {
  const f32x4_t v = *(const gf32x4*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gstore4(gfloat* p, float4 v) { *(gf32x4*)p = f32x4_t{v.x, v.y, v.z, v.w}; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over the block (blockDim.x threads, multiple of 64); result in every thread.
__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// 16-byte weight chunk: 8 bf16 or 4 fp32 values.
template <typename WT>
struct Chunk;
template <>
struct Chunk<uint16_t> {
  static constexpr int N = 8;
  uint4 raw;
  __device__ __forceinline__ void load(const uint16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float dot(const float* x) const {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(w[i] << 16), x[2 * i], s);
      s = fmaf(__uint_as_float(w[i] & 0xFFFF0000u), x[2 * i + 1], s);
    }
    return s;
  }
};
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  float4 raw;
  __device__ __forceinline__ void load(const float* p) { raw = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float dot(const float* x) const {
    float s = raw.x * x[0];
    s = fmaf(raw.y, x[1], s);
    s = fmaf(raw.z, x[2], s);
    return fmaf(raw.w, x[3], s);
  }
};

template <typename WT>
__device__ __forceinline__ float load_w(const WT* p, size_t i);
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float load_w<float>(const float* p, size_t i) { return p[i]; }

__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}

// ------------------------------------------------------------------ embed

template <typename WT>
__global__ __launch_bounds__(256) void embed_prefill_kernel(const WT* __restrict__ E, int H,
                                                             const int32_t* __restrict__ ids,
                                                             const float* __restrict__ audio, int a0, int La,
                                                             float* __restrict__ X, float* __restrict__ ssq) {
  __shared__ float red[8];
  const int t = blockIdx.x;
  float* out = X + (size_t)t * H;
  float ss = 0.f;
  if (t >= a0 && t < a0 + La) {
    const float* src = audio + (size_t)(t - a0) * H;
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
      const float v = src[i];
      out[i] = v;
      ss = fmaf(v, v, ss);
    }
  } else {
    const WT* row = E + (size_t)ids[t] * H;
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
      const float v = load_w(row, i);
      out[i] = v;
      ss = fmaf(v, v, ss);
    }
  }
  if (ssq) {
    ss = block_sum(ss, red);
    if (threadIdx.x == 0) ssq[t] = ss;
  }
}

// One row per state of a batched decode step: X[r] = E[tok[r]].
template <typename WT>
__global__ __launch_bounds__(256) void embed_rows_kernel(const WT* __restrict__ E, int H, BatchRows rows,
                                                          float* __restrict__ X, float* __restrict__ ssq) {
  __shared__ float red[8];
  const int r = blockIdx.x;
  const WT* src = E + (size_t)rows.tok[r] * H;
  float* out = X + (size_t)r * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float v = load_w(src, i);
    out[i] = v;
    ss = fmaf(v, v, ss);
  }
  if (ssq) {
    ss = block_sum(ss, red);
    if (threadIdx.x == 0) ssq[r] = ss;
  }
}

// LM head over the tied embedding with fused final RMSNorm and greedy argmax.
template <typename WT, int ROWS, int KCH>
__global__ __launch_bounds__(256) void lm_head_kernel(const WT* __restrict__ E, int V, int K,
                                                       const float* __restrict__ xin,
                                                       const float* __restrict__ gain, float eps,
                                                       float* __restrict__ logits, unsigned long long* key) {
  extern __shared__ float smem[];
  float* xs = smem;
  float* red = smem + K;
  __shared__ unsigned long long bkey[4];
  constexpr int VN = Chunk<WT>::N;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float ss = 0.f;
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    float v = xin[i];
    ss = fmaf(v, v, ss);
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)K + eps);
  for (int i = threadIdx.x; i < K; i += blockDim.x) xs[i] = xin[i] * inv * gain[i];
  __syncthreads();

  const int r0 = (blockIdx.x * 4 + wave) * ROWS;
  const int nch = K / VN;
  Chunk<WT> w[KCH][ROWS];
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = lane + kWave * j;
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      if (c < nch && r0 + r < V) w[j][r].load(E + (size_t)(r0 + r) * K + (size_t)c * VN);
  }
  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = lane + kWave * j;
    if (c < nch) {
      float xv[VN];
#pragma unroll
      for (int i = 0; i < VN; ++i) xv[i] = xs[c * VN + i];
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
        if (r0 + r < V) acc[r] += w[j][r].dot(xv);
    }
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float v = wave_sum(acc[r]);
    const int row = r0 + r;
    if (row < V) {
      if (logits && lane == r) logits[row] = v;
      const unsigned long long k = argmax_key(v, row);
      best = k > best ? k : best;
    }
  }
  if (lane == 0) bkey[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long b = bkey[0];
    for (int i = 1; i < 4; ++i) b = bkey[i] > b ? bkey[i] : b;
    atomicMax(key + blockIdx.x % kKeySlots, b);
  }
}

__global__ void argmax_final_kernel(const unsigned long long* key, int n, int32_t* out) {
  const int i = threadIdx.x;
  if (i < n) {
    unsigned long long b = key[i * kKeySlots];
    for (int s = 1; s < kKeySlots; ++s) b = key[i * kKeySlots + s] > b ? key[i * kKeySlots + s] : b;
    out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
  }
}

// key[r] = max over v of argmax_key(logits[r][v], v); grid (chunks, rows).
__global__ __launch_bounds__(256) void argmax_rows_kernel(const float* __restrict__ logits, int V,
                                                           unsigned long long* key) {
  __shared__ unsigned long long wbest[4];
  const int r = blockIdx.y;
  const float* lr = logits + (size_t)r * V;
  unsigned long long best = 0ull;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < V; i += gridDim.x * blockDim.x) {
    const unsigned long long k = argmax_key(lr[i], i);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long k = __shfl_xor(best, o, kWave);
    best = k > best ? k : best;
  }
  if (threadIdx.x % kWave == 0) wbest[threadIdx.x / kWave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x / kWave); ++w) best = wbest[w] > best ? wbest[w] : best;
    atomicMax(key + r * kKeySlots + blockIdx.x % kKeySlots, best);
  }
}

__global__ void reset_keys_kernel(unsigned long long* key, int n) {
  for (int i = threadIdx.x; i < n * kKeySlots; i += blockDim.x) key[i] = 0ull;
}

// ------------------------------------------ per-head Q/K RMSNorm + RoPE + KV append
// One wave per (row, head); heads [0, NQ) are query heads, [NQ, NQ+NKV) key
// heads (which also copy the matching V head). Lane l < D/2 owns the rotate-
// half pair (l, l + D/2). Q and K are rewritten in place (post-RoPE); K and V
// of position pos0 + row go to the paged cache.

__device__ __forceinline__ void qk_rope_row(float* __restrict__ qrow, int head, int pos, int NQ, int NKV, int D,
                                            int L, float eps, const float* __restrict__ q_norm,
                                            const float* __restrict__ k_norm, const float* __restrict__ rcos,
                                            const float* __restrict__ rsin, const int64_t* __restrict__ page_table,
                                            int layer) {
  const int lane = threadIdx.x;
  const int half = D / 2;
  const bool is_q = head < NQ;
  float* vec = qrow + (size_t)head * D;  // q heads then k heads are contiguous
  const float* g = is_q ? q_norm : k_norm;
  float a = 0.f, b = 0.f;
  if (lane < half) {
    a = vec[lane];
    b = vec[lane + half];
  }
  const float ss = wave_sum(a * a + b * b);
  const float inv = 1.f / sqrtf(ss / (float)D + eps);
  if (lane < half) {
    a = a * inv * g[lane];
    b = b * inv * g[lane + half];
    const float c = rcos[(size_t)pos * half + lane], s = rsin[(size_t)pos * half + lane];
    const float ra = a * c - b * s, rb = b * c + a * s;
    vec[lane] = ra;
    vec[lane + half] = rb;
    if (!is_q) {
      const int kh = head - NQ;
      Dims d{L, 0, NQ, NKV, D, 0, 0, 0.f};
      gfloat* page = page_at(page_table, pos / kPage);
      const int slot = pos % kPage;
      gfloat* kd = page + page_offset(d, layer, 0, kh, slot);
      gfloat* vd = page + page_offset(d, layer, 1, kh, slot);
      const float* vs = qrow + (size_t)(NQ + NKV + kh) * D;
      kd[lane] = ra;
      kd[lane + half] = rb;
      vd[lane] = vs[lane];
      vd[lane + half] = vs[lane + half];
    }
  }
}

// Several heads per wave for head_dim D (32, 64 or 128): LPH = D / 8 lanes
// per head, lane j of a head owning the float4 groups [4 j, 4 j + 4) and
// [D/2 + 4 j, D/2 + 4 j + 4) (rotate-half partners), so one wave covers
// 64 / LPH heads of a row with 16-byte accesses. Same arithmetic per element
// as qk_rope_row; the sum of squares is reduced over the head's LPH lanes.
template <int D>
__global__ __launch_bounds__(256) void qk_rope_append_vec_kernel(float* __restrict__ qkv, int ld, int pos0, int NQ,
                                                                  int NKV, int L, float eps,
                                                                  const float* __restrict__ q_norm,
                                                                  const float* __restrict__ k_norm,
                                                                  const float* __restrict__ rcos,
                                                                  const float* __restrict__ rsin,
                                                                  const int64_t* __restrict__ page_table, int layer) {
  constexpr int HALF = D / 2, LPH = D / 8, HPW = kWave / LPH;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int row = blockIdx.y, j = lane % LPH;
  const int head = (blockIdx.x * 4 + wave) * HPW + lane / LPH;
  const bool live = head < NQ + NKV;
  const int hd = live ? head : NQ + NKV - 1;  // idle lanes mirror a real head, store nothing
  const int pos = pos0 + row;
  const bool is_q = hd < NQ;
  float* rowp = qkv + (size_t)row * ld;
  float* vec = rowp + (size_t)hd * D;
  const float* g = is_q ? q_norm : k_norm;
  float4 a = *reinterpret_cast<const float4*>(vec + 4 * j);
  float4 b = *reinterpret_cast<const float4*>(vec + HALF + 4 * j);
  float ss = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
#pragma unroll
  for (int o = 1; o < LPH; o <<= 1) ss += __shfl_xor(ss, o, kWave);
  const float inv = 1.f / sqrtf(ss / (float)D + eps);
  const float4 ga = *reinterpret_cast<const float4*>(g + 4 * j);
  const float4 gb = *reinterpret_cast<const float4*>(g + HALF + 4 * j);
  const float4 c = *reinterpret_cast<const float4*>(rcos + (size_t)pos * HALF + 4 * j);
  const float4 sn = *reinterpret_cast<const float4*>(rsin + (size_t)pos * HALF + 4 * j);
  float av[4] = {a.x * inv * ga.x, a.y * inv * ga.y, a.z * inv * ga.z, a.w * inv * ga.w};
  float bv[4] = {b.x * inv * gb.x, b.y * inv * gb.y, b.z * inv * gb.z, b.w * inv * gb.w};
  const float cv[4] = {c.x, c.y, c.z, c.w}, sv[4] = {sn.x, sn.y, sn.z, sn.w};
  float ra[4], rb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = av[e] * cv[e] - bv[e] * sv[e];
    rb[e] = bv[e] * cv[e] + av[e] * sv[e];
  }
  if (!live) return;
  const float4 ra4 = make_float4(ra[0], ra[1], ra[2], ra[3]), rb4 = make_float4(rb[0], rb[1], rb[2], rb[3]);
  *reinterpret_cast<float4*>(vec + 4 * j) = ra4;
  *reinterpret_cast<float4*>(vec + HALF + 4 * j) = rb4;
  if (!is_q) {
    const int kh = hd - NQ;
    Dims d{L, 0, NQ, NKV, D, 0, 0, 0.f};
    gfloat* page = page_at(page_table, pos / kPage);
    const int slot = pos % kPage;
    gfloat* kd = page + page_offset(d, layer, 0, kh, slot);
    gfloat* vd = page + page_offset(d, layer, 1, kh, slot);
    const float* vs = rowp + (size_t)(NQ + NKV + kh) * D;
    gstore4(kd + 4 * j, ra4);
    gstore4(kd + HALF + 4 * j, rb4);
    gstore4(vd + 4 * j, *reinterpret_cast<const float4*>(vs + 4 * j));
    gstore4(vd + HALF + 4 * j, *reinterpret_cast<const float4*>(vs + HALF + 4 * j));
  }
}

// Prompt rows: row t sits at position pos0 + t of one state.
__global__ __launch_bounds__(64) void qk_rope_append_kernel(float* __restrict__ qkv, int ld, int pos0, int NQ,
                                                             int NKV, int D, int L, float eps,
                                                             const float* __restrict__ q_norm,
                                                             const float* __restrict__ k_norm,
                                                             const float* __restrict__ rcos,
                                                             const float* __restrict__ rsin,
                                                             const int64_t* __restrict__ page_table, int layer) {
  const int row = blockIdx.y;
  qk_rope_row(qkv + (size_t)row * ld, blockIdx.x, pos0 + row, NQ, NKV, D, L, eps, q_norm, k_norm, rcos, rsin,
              page_table, layer);
}

// ------------------------------------------------ short prompts: fused attention
// Causal prefill attention for prompts of at most kSmallT positions, with
// the per-head Q/K-RMSNorm, RoPE and the K/V append of the same layer
// folded in (one launch instead of three). Block = (KV head g, block of
// kSmallQB query rows [q0, q1)), 8 waves. Every thread owns one rotation pair (i,
// i + D / 2) of one row per pass; a pass's loads are all issued before any
// is used, and a row's sum of squares is reduced over its D / 2 lanes. The
// block prepares the keys [0, q1) in LDS (keys of earlier blocks are
// recomputed, not exchanged) and appends K/V of its own rows [q0, q1) to the
// state's pages. Each (query row, query head of the group) is then one
// wave's item: scores with one lane per key, the softmax in base 2 (q
// carries log2(e) / sqrt(D)), and the output with each lane holding D / 64
// dimensions. All in fp32.
template <int HALF>
__device__ __forceinline__ float pair_sum(float v) {
#pragma unroll
  for (int o = 1; o < HALF; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// query rows per block: 2 rows of a 48-token prompt give 192 blocks (8 rows:
// 48); the keys each block prepares are recomputed, not shared (48-token
// prefill 1.72 -> 1.61 ms; one row per block: 1.64 ms)
constexpr int kSmallQB = 2;
template <int D, int GROUP>
__global__ __launch_bounds__(512) void attn_small_kernel(const float* __restrict__ qkv, int T, int NQ, int NKV,
                                                          int L, float eps, float qscale,
                                                          const float* __restrict__ q_norm,
                                                          const float* __restrict__ k_norm,
                                                          const float* __restrict__ rcos,
                                                          const float* __restrict__ rsin,
                                                          const int64_t* __restrict__ page_table, int layer,
                                                          float* __restrict__ out) {
  constexpr int HALF = D / 2, QB = kSmallQB, KP = D + 1;  // K rows padded: lane-per-key reads hit distinct banks
  constexpr int NW = 8, RPP = 512 / HALF;          // waves; rows per pass
  constexpr int DPL = (D + kWave - 1) / kWave;     // output dimensions per lane
  constexpr int KPASS = (kSmallT + RPP - 1) / RPP;
  __shared__ float kl[kSmallT * KP];
  __shared__ float vl[kSmallT * D];
  __shared__ float ql[QB * GROUP * D];
  __shared__ float pl[NW][kSmallT];
  const int g = blockIdx.x, q0 = blockIdx.y * QB, q1 = min(T, q0 + QB);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int pi = threadIdx.x % HALF, pr = threadIdx.x / HALF;  // this thread's pair and row within a pass
  const int ld = (NQ + 2 * NKV) * D;
  Dims d{L, 0, NQ, NKV, D, 0, 0, 0.f};
  const float gk0 = k_norm[pi], gk1 = k_norm[pi + HALF];

  // keys and values [0, q1)
  {
    float k0[KPASS], k1[KPASS], v0[KPASS], v1[KPASS], c[KPASS], sn[KPASS];
#pragma unroll
    for (int ps = 0; ps < KPASS; ++ps) {
      const int t = min(ps * RPP + pr, q1 - 1);  // rows past q1 repeat the last one, stored nowhere
      const float* row = qkv + (size_t)t * ld;
      k0[ps] = row[(size_t)(NQ + g) * D + pi];
      k1[ps] = row[(size_t)(NQ + g) * D + pi + HALF];
      v0[ps] = row[(size_t)(NQ + NKV + g) * D + pi];
      v1[ps] = row[(size_t)(NQ + NKV + g) * D + pi + HALF];
      c[ps] = rcos[(size_t)t * HALF + pi];
      sn[ps] = rsin[(size_t)t * HALF + pi];
    }
#pragma unroll
    for (int ps = 0; ps < KPASS; ++ps) {
      const int t = ps * RPP + pr;
      const float inv = 1.f / sqrtf(pair_sum<HALF>(k0[ps] * k0[ps] + k1[ps] * k1[ps]) / (float)D + eps);
      const float x0 = k0[ps] * inv * gk0, x1 = k1[ps] * inv * gk1;
      const float r0 = x0 * c[ps] - x1 * sn[ps], r1 = x1 * c[ps] + x0 * sn[ps];
      if (t < q1) {
        kl[t * KP + pi] = r0;
        kl[t * KP + pi + HALF] = r1;
        vl[t * D + pi] = v0[ps];
        vl[t * D + pi + HALF] = v1[ps];
        if (t >= q0) {
          gfloat* page = page_at(page_table, t / kPage);
          gfloat* kd = page + page_offset(d, layer, 0, g, t % kPage);
          gfloat* vd = page + page_offset(d, layer, 1, g, t % kPage);
          kd[pi] = r0;
          kd[pi + HALF] = r1;
          vd[pi] = v0[ps];
          vd[pi + HALF] = v1[ps];
        }
      }
    }
  }
  // the group's query heads of rows [q0, q1), scaled for base-2 scores
  {
    constexpr int QPASS = (QB * GROUP + RPP - 1) / RPP;
    const float gq0 = q_norm[pi], gq1 = q_norm[pi + HALF];
    float a0[QPASS], a1[QPASS], c[QPASS], sn[QPASS];
#pragma unroll
    for (int ps = 0; ps < QPASS; ++ps) {
      const int it = min(ps * RPP + pr, (q1 - q0) * GROUP - 1);
      const int t = q0 + it / GROUP, hh = it % GROUP;
      const float* src = qkv + (size_t)t * ld + (size_t)(g * GROUP + hh) * D;
      a0[ps] = src[pi];
      a1[ps] = src[pi + HALF];
      c[ps] = rcos[(size_t)t * HALF + pi];
      sn[ps] = rsin[(size_t)t * HALF + pi];
    }
#pragma unroll
    for (int ps = 0; ps < QPASS; ++ps) {
      const int it = ps * RPP + pr;
      const float inv = 1.f / sqrtf(pair_sum<HALF>(a0[ps] * a0[ps] + a1[ps] * a1[ps]) / (float)D + eps);
      const float x0 = a0[ps] * inv * gq0, x1 = a1[ps] * inv * gq1;
      if (it < (q1 - q0) * GROUP) {
        ql[it * D + pi] = (x0 * c[ps] - x1 * sn[ps]) * qscale;
        ql[it * D + pi + HALF] = (x1 * c[ps] + x0 * sn[ps]) * qscale;
      }
    }
  }
  __syncthreads();

  for (int it = wave; it < (q1 - q0) * GROUP; it += NW) {
    const int t = q0 + it / GROUP, hh = it % GROUP;
    const float* q = ql + it * D;
    // scores: lane u <-> key u (keys past t masked)
    float sc = -INFINITY;
    if (lane <= t) {
      float a = 0.f;
#pragma unroll 16
      for (int e = 0; e < D; ++e) a = fmaf(q[e], kl[lane * KP + e], a);
      sc = a;
    }
    const float mx = wave_max(sc);
    const float pv = lane <= t ? __builtin_amdgcn_exp2f(sc - mx) : 0.f;
    const float ls = wave_sum(pv);
    pl[wave][lane] = pv;
    __builtin_amdgcn_wave_barrier();
    float o[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    for (int u = 0; u <= t; ++u) {
      const float pu = pl[wave][u];
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        if (lane + k * kWave < D) o[k] = fmaf(pu, vl[u * D + lane + k * kWave], o[k]);
    }
    float* dst = out + (size_t)t * NQ * D + (size_t)(g * GROUP + hh) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      if (lane + k * kWave < D) dst[lane + k * kWave] = o[k] / ls;
    __builtin_amdgcn_wave_barrier();  // pl is rewritten by this wave's next item
  }
}

// ------------------------------------------------ batched decode attention
// One launch per layer for the rows of a batched decode step; row r is one
// state at position pos_r. Block = (kv head g, split s of kAttnChunk
// positions, row r), 4 waves; blocks are numbered kv head fastest, so with
// 8 KV heads every block of head g runs on XCD g and rows that share prompt
// pages (clones) read them through one L2.
//  1. Prologue: per-head Q/K-RMSNorm and RoPE at pos_r of the GROUP query
//     heads and of key head g (one wave per head), into LDS. The block whose
//     split holds pos_r also appends K/V at pos_r to the row's pages and uses
//     its LDS copy for that key.
//  2. Split-K flash decoding over [u0, u1) of the row's pages: lane = 8 slot +
//     part, 8 keys at a time, head_dim split over 8 lanes, the next 8 keys in
//     flight while the current ones are used; the GROUP query heads share every
//     K/V load. Scores are in base 2 (q carries log2(e) / sqrt(D)).
//  3. Merge: with one split the block writes the output; otherwise each block
//     publishes (m, l, o) as tagged device-scope words and bumps the (row,
//     kv head) counter, and the last block to arrive merges all splits in
//     split order (scheduling-independent), writes the output and resets the
//     counter.
constexpr unsigned long long kAttnWaitTicks = 200000000ull;  // about 0.1 s of s_memtime

template <int D, int GROUP>
__global__ __launch_bounds__(256) void attn_rows_kernel(AttnRows a) {
  constexpr int DPL = D / 8;
  constexpr int HALF = D / 2;
  __shared__ float q_l[GROUP][D], k_l[D], v_l[D];
  __shared__ float sm_m[4][GROUP], sm_l[4][GROUP];
  __shared__ float sm_o[4][GROUP][D];
  __shared__ const gfloat* pg[kAttnChunk / kPage];
  __shared__ int s_last;
  const int g = blockIdx.x, s = blockIdx.y, r = blockIdx.z, nsplit = gridDim.y;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int slot = lane / 8, part = lane % 8;
  const int pos = a.rows.pos[r];
  const int n = pos + 1;
  const int64_t* __restrict__ page_table = a.rows.pt[r];
  const int u0 = s * kAttnChunk, u1 = min(n, u0 + kAttnChunk);
  const bool has_cur = u0 <= pos && pos < u1;
  const int NQ = a.NKV * GROUP;
  Dims d{a.L, 0, NQ, a.NKV, D, 0, 0, 0.f};
  float* row = a.qkv + (size_t)r * a.ld;

  // the split's page pointers, so that each key load needs no dependent
  // global load first
  if (threadIdx.x < kAttnChunk / kPage && u0 < u1)
    pg[threadIdx.x] = page_at(page_table, min(u0 / kPage + (int)threadIdx.x, (u1 - 1) / kPage));

  // 1. QK-norm + RoPE: items 0..GROUP-1 are the query heads, GROUP the key head
  for (int it = wave; it <= GROUP; it += 4) {
    const bool is_q = it < GROUP;
    const float* src = row + (size_t)(is_q ? g * GROUP + it : NQ + g) * D;
    const float* gain = is_q ? a.q_norm : a.k_norm;
    float x0 = 0.f, x1 = 0.f;
    if (lane < HALF) {
      x0 = src[lane];
      x1 = src[lane + HALF];
    }
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
    if (lane < HALF) {
      x0 = x0 * inv * gain[lane];
      x1 = x1 * inv * gain[lane + HALF];
      const float c = a.rcos[(size_t)pos * HALF + lane], sn = a.rsin[(size_t)pos * HALF + lane];
      const float r0 = x0 * c - x1 * sn, r1 = x1 * c + x0 * sn;
      if (is_q) {
        q_l[it][lane] = r0 * a.qscale;
        q_l[it][lane + HALF] = r1 * a.qscale;
      } else {
        k_l[lane] = r0;
        k_l[lane + HALF] = r1;
        const float* vs = row + (size_t)(NQ + a.NKV + g) * D;
        const float v0 = vs[lane], v1 = vs[lane + HALF];
        v_l[lane] = v0;
        v_l[lane + HALF] = v1;
        if (has_cur) {
          gfloat* page = page_at(page_table, pos / kPage);
          gfloat* kd = page + page_offset(d, a.layer, 0, g, pos % kPage);
          gfloat* vd = page + page_offset(d, a.layer, 1, g, pos % kPage);
          kd[lane] = r0;
          kd[lane + HALF] = r1;
          vd[lane] = v0;
          vd[lane + HALF] = v1;
        }
      }
    }
  }
  __syncthreads();

  float qr[GROUP][DPL];
#pragma unroll
  for (int h = 0; h < GROUP; ++h)
#pragma unroll
    for (int i = 0; i < DPL; ++i) qr[h][i] = q_l[h][part * DPL + i];

  float m[GROUP], l[GROUP], acc[GROUP][DPL];
#pragma unroll
  for (int h = 0; h < GROUP; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[h][i] = 0.f;
  }

  // 2. key u clamped into [u0, u1): loads past the end repeat the last key
  // and are masked out; the key at pos comes from LDS
  auto load = [&](int base, float (&kv)[DPL], float (&vv)[DPL]) {
    const int u = min(base + slot, u1 - 1);
    const gfloat* page = pg[u / kPage - u0 / kPage];
    const gfloat* kp = page + page_offset(d, a.layer, 0, g, u % kPage) + part * DPL;
    const gfloat* vp = page + page_offset(d, a.layer, 1, g, u % kPage) + part * DPL;
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const float4 x = gload4(kp + i);
      kv[i] = x.x; kv[i + 1] = x.y; kv[i + 2] = x.z; kv[i + 3] = x.w;
      const float4 y = gload4(vp + i);
      vv[i] = y.x; vv[i + 1] = y.y; vv[i + 2] = y.z; vv[i + 3] = y.w;
    }
  };

  // One step: the wave's 8 keys from base, already in (kc, vc).
  auto step = [&](int base, float (&kc)[DPL], float (&vc)[DPL]) __attribute__((always_inline)) {
    const int u = base + slot;
    const bool valid = u < u1;
    // the key at pos (its page store may not be visible yet) from LDS
    if (base <= pos && pos < base + 8 && u == pos) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        kc[i] = k_l[part * DPL + i];
        vc[i] = v_l[part * DPL + i];
      }
    }
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
      float sc = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) sc = fmaf(qr[h][i], kc[i], sc);
      sc += __shfl_xor(sc, 1, kWave);
      sc += __shfl_xor(sc, 2, kWave);
      sc += __shfl_xor(sc, 4, kWave);
      if (!valid) sc = -INFINITY;
      float mx = fmaxf(sc, __shfl_xor(sc, 8, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mn = fmaxf(m[h], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
      const float p = valid ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
      float ps = p + __shfl_xor(p, 8, kWave);
      ps += __shfl_xor(ps, 16, kWave);
      ps += __shfl_xor(ps, 32, kWave);
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[h][i] = fmaf(p, vc[i], acc[h][i] * alpha);
      m[h] = mn;
    }
  };
  // the wave's steps (at most kAttnChunk / 32) unrolled over two register
  // sets, so the next step's loads stay in flight while the current one is
  // used (a rolling copy from one set into the other would wait for them).
  // The loads are unconditional (clamped keys) so that the wait before each
  // step covers only that step's loads.
  constexpr int NIT = kAttnChunk / 32;
  const int b0 = u0 + wave * 8;
  if (u0 < u1) {
    float kA[DPL], vA[DPL], kB[DPL], vB[DPL];
    load(b0, kA, vA);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int base = b0 + 32 * it;
      if (base >= u1) break;
      // (the scheduler would otherwise sink the next loads below the step)
      if (it % 2 == 0) {
        if (it + 1 < NIT) load(base + 32, kB, vB);
        __builtin_amdgcn_sched_barrier(0);
        step(base, kA, vA);
      } else {
        if (it + 1 < NIT) load(base + 32, kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        step(base, kB, vB);
      }
    }
  }
  // sum the 8 key slots (same running max within the wave)
#pragma unroll
  for (int h = 0; h < GROUP; ++h)
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float v = acc[h][i];
      v += __shfl_xor(v, 8, kWave);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[h][i] = v;
    }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < GROUP; ++h)
#pragma unroll
      for (int i = 0; i < DPL; ++i) sm_o[wave][h][part * DPL + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  // 3. the 4 waves' (m, l, o) merged in wave order; thread -> (head, dim)
  float* out = a.out + (size_t)r * NQ * D + (size_t)g * GROUP * D;
  const unsigned long long tag = (unsigned long long)a.tag << 32;
  unsigned long long* words = a.part + ((size_t)r * a.NKV + g) * nsplit * GROUP * (D + 2);
  for (int idx = threadIdx.x; idx < GROUP * D; idx += blockDim.x) {
    const int h = idx / D, i = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, ls = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = sm_m[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[w][h] - M);
      o = fmaf(f, sm_o[w][h][i], o);
      ls = fmaf(f, sm_l[w][h], ls);
    }
    if (nsplit == 1) {
      out[(size_t)h * D + i] = o / ls;
    } else {
      unsigned long long* wd = words + ((size_t)s * GROUP + h) * (D + 2);
      __hip_atomic_store(wd + 2 + i, tag | __float_as_uint(o), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (i == 0) {
        __hip_atomic_store(wd, tag | __float_as_uint(M), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(wd + 1, tag | __float_as_uint(ls), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (nsplit == 1) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned* cnt = a.cnt + (size_t)r * a.NKV + g;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(nsplit - 1);
  __syncthreads();
  if (!s_last) return;
  // every split's (m, l, o_i) requested at once, 8 splits per round
  // (addresses clamped to the last split, surplus ignored); a word not yet
  // visible is re-read under a time limit
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  bool late = false;
  auto value = [&](unsigned long long w, const unsigned long long* p) {
    while ((w >> 32) != a.tag && !late) {
      late = __builtin_amdgcn_s_memtime() - t0 > kAttnWaitTicks;
      w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return (w >> 32) == a.tag ? __uint_as_float((unsigned)w) : __builtin_nanf("");
  };
  for (int idx = threadIdx.x; idx < GROUP * D; idx += blockDim.x) {
    const int h = idx / D, i = idx % D;
    float M = -INFINITY, o = 0.f, ls = 0.f;
    for (int sb = 0; sb < nsplit; sb += 8) {
      unsigned long long wm[8], wl[8], wo[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const unsigned long long* wd = words + ((size_t)min(sb + u, nsplit - 1) * GROUP + h) * (D + 2);
        wm[u] = __hip_atomic_load(wd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wl[u] = __hip_atomic_load(wd + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wo[u] = __hip_atomic_load(wd + 2 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (sb + u < nsplit) {
          const unsigned long long* wd = words + ((size_t)(sb + u) * GROUP + h) * (D + 2);
          const float ms = value(wm[u], wd), lv = value(wl[u], wd + 1), ov = value(wo[u], wd + 2 + i);
          // running merge in split order
          const float Mn = fmaxf(M, ms);
          const float fa = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
          const float fb = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - Mn);
          o = o * fa + ov * fb;
          ls = ls * fa + lv * fb;
          M = Mn;
        }
      }
    }
    out[(size_t)h * D + i] = o / ls;
  }
  if (late) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------ prefill attention
// Causal GQA flash attention in fp32 on the vector units. Block = (query
// tile of QT positions, kv head g); its 64 query rows are the GROUP heads x QT
// positions, 4 threads per row. Thread part p owns the float4 chunks
// c = 4 i + p of head_dim. K/V tiles of 32 keys are staged in LDS.

template <int D, int GROUP>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const float* __restrict__ qkv, int T, int ld, int NQ,
                                                            int NKV, float* __restrict__ out, int ldo,
                                                            float scale) {
  constexpr int QT = 64 / GROUP;
  constexpr int KT = 32;
  constexpr int NC = D / 16;  // float4 chunks per thread
  __shared__ float4 Ks[KT][D / 4];
  __shared__ float4 Vs[KT][D / 4];
  const int g = blockIdx.y;
  const int t0 = blockIdx.x * QT;
  const int row = threadIdx.x / 4, part = threadIdx.x % 4;
  const int hh = row / QT, tq = row % QT;
  const int t = t0 + tq;
  const int h = g * GROUP + hh;
  const bool active = t < T;

  float4 q[NC], o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    o[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    q[c] = active ? *reinterpret_cast<const float4*>(qkv + (size_t)t * ld + (size_t)h * D + (c * 4 + part) * 4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    q[c].x *= scale; q[c].y *= scale; q[c].z *= scale; q[c].w *= scale;
  }
  float m = -INFINITY, l = 0.f;
  const int t_last = min(T, t0 + QT) - 1;
  const size_t koff = (size_t)NQ * D + (size_t)g * D;
  const size_t voff = (size_t)(NQ + NKV) * D + (size_t)g * D;
  for (int k0 = 0; k0 <= t_last; k0 += KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < KT * D / 4; idx += blockDim.x) {
      const int kr = idx / (D / 4), kc = idx % (D / 4);
      const int u = k0 + kr;
      if (u < T) {
        Ks[kr][kc] = *reinterpret_cast<const float4*>(qkv + (size_t)u * ld + koff + kc * 4);
        Vs[kr][kc] = *reinterpret_cast<const float4*>(qkv + (size_t)u * ld + voff + kc * 4);
      } else {
        Ks[kr][kc] = make_float4(0.f, 0.f, 0.f, 0.f);
        Vs[kr][kc] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __syncthreads();
    float s[KT];
    float mx = m;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 kk = Ks[j][c * 4 + part];
        a = fmaf(q[c].x, kk.x, a);
        a = fmaf(q[c].y, kk.y, a);
        a = fmaf(q[c].z, kk.z, a);
        a = fmaf(q[c].w, kk.w, a);
      }
      a += __shfl_xor(a, 1, kWave);
      a += __shfl_xor(a, 2, kWave);
      s[j] = (k0 + j <= t) ? a : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    if (mx == -INFINITY) continue;  // inactive row (t >= T): nothing visible yet
    const float alpha = expf(m - mx);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      o[c].x *= alpha; o[c].y *= alpha; o[c].z *= alpha; o[c].w *= alpha;
    }
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const float p = (s[j] == -INFINITY) ? 0.f : expf(s[j] - mx);
      l += p;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 vv = Vs[j][c * 4 + part];
        o[c].x = fmaf(p, vv.x, o[c].x);
        o[c].y = fmaf(p, vv.y, o[c].y);
        o[c].z = fmaf(p, vv.z, o[c].z);
        o[c].w = fmaf(p, vv.w, o[c].w);
      }
    }
    m = mx;
  }
  if (active) {
    const float il = 1.f / l;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float4 r = o[c];
      r.x *= il; r.y *= il; r.z *= il; r.w *= il;
      *reinterpret_cast<float4*>(out + (size_t)t * ldo + (size_t)h * D + (c * 4 + part) * 4) = r;
    }
  }
}

// Causal GQA flash attention on the matrix cores, head_dim 128. Block = (64
// query positions, kv head g), 4 waves; wave w owns positions q0 + 16 w + i
// (i < 16) of all GROUP query heads of g. Per key tile of KT the block stages
// K as [key][d] and V transposed as [d][key] in LDS, each as bf16 hi + lo
// (hi = bf16(x), lo = bf16(x - hi)). Scores are computed transposed,
// S^T = K Q^T, so that a lane holds the scores of one query (column l % 16)
// for keys 16 j + 4 (l / 16) + e: that is both where the online softmax needs
// them (row statistics are per lane, reduced over the 4 lanes of the query)
// and, once exponentiated, the B operand of O^T = V^T P^T, whose k-slots are
// taken as keys {4 (l / 16) + e} and {16 + 4 (l / 16) + e} of each 32-key
// group (the A operand reads V^T at the same keys). Every product is the sum
// of three bf16 MFMAs (hi hi, hi lo, lo hi), about 16 mantissa bits. Scores
// are kept in base 2 (Q carries log2(e) / sqrt(D)), so the softmax uses the
// hardware exp2.
// K and V of one KV head for the matrix-core attention, converted once per
// layer: kh / kl [g][t][128] bf16 hi / lo of the rotated keys, vth / vtl
// [g][128][Tp] bf16 hi / lo of the values transposed (columns t >= T repeat
// row T - 1, so every staged tile is finite). Within each 32-key group the
// V^T columns are stored in the order the P^T operand takes its k-slots:
// keys 4 q + e and 16 + 4 q + e (e = 0..3) at slots 8 q + e and 8 q + 4 + e,
// so a lane's A operand of O^T = V^T P^T is one 16-byte LDS read. Block =
// (32 tokens, head g): at 1024 tokens that is 256 blocks. With rp.norm set the keys arrive as projected: the
// block applies the K-RMSNorm and RoPE of each key (the arithmetic of
// qk_rope_append_vec_kernel) and appends K and V of positions rp.pos0 + t to
// the state's pages.
constexpr int kKvTile = 32;  // tokens per kv_split block (one 32-key group)
__global__ __launch_bounds__(256) void kv_split_kernel(const float* __restrict__ qkv, int T, int ld, int NQ,
                                                        int NKV, uint16_t* __restrict__ kh,
                                                        uint16_t* __restrict__ kl, uint16_t* __restrict__ vth,
                                                        uint16_t* __restrict__ vtl, int Tp, QkRope rp) {
  constexpr int D = 128, TT = kKvTile, HALF = D / 2;
  __shared__ float vs[D][TT + 1];
  const int g = blockIdx.y, t0 = blockIdx.x * TT;
  const float* kbase = qkv + (size_t)(NQ + g) * D;
  const float* vbase = qkv + (size_t)(NQ + NKV + g) * D;
#pragma unroll
  for (int i = 0; i < TT * D / 4 / 256; ++i) {
    // 32 threads per key (one half-wave), thread c % 32 holding columns d0..d0+3
    const int c = threadIdx.x + 256 * i, tl = c / (D / 4), d0 = 4 * (c % (D / 4));
    const int t = min(t0 + tl, T - 1);
    float4 k = *reinterpret_cast<const float4*>(kbase + (size_t)t * ld + d0);
    const float4 v = *reinterpret_cast<const float4*>(vbase + (size_t)t * ld + d0);
    if (rp.norm) {
      // rotate-half partner columns d0 +- 64 sit 16 lanes away
      float ss = k.x * k.x + k.y * k.y + k.z * k.z + k.w * k.w;
#pragma unroll
      for (int o = 1; o < D / 4; o <<= 1) ss += __shfl_xor(ss, o, kWave);
      const float inv = 1.f / sqrtf(ss / (float)D + rp.eps);
      const float4 gk = *reinterpret_cast<const float4*>(rp.k_norm + d0);
      const float x[4] = {k.x * inv * gk.x, k.y * inv * gk.y, k.z * inv * gk.z, k.w * inv * gk.w};
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __shfl_xor(x[e], 16, kWave);
      const int pos = rp.pos0 + t, j0 = d0 % HALF;
      const float4 cs = *reinterpret_cast<const float4*>(rp.rcos + (size_t)pos * HALF + j0);
      const float4 sn = *reinterpret_cast<const float4*>(rp.rsin + (size_t)pos * HALF + j0);
      const float cv[4] = {cs.x, cs.y, cs.z, cs.w}, sv[4] = {sn.x, sn.y, sn.z, sn.w};
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r[e] = d0 < HALF ? x[e] * cv[e] - y[e] * sv[e] : x[e] * cv[e] + y[e] * sv[e];
      k = make_float4(r[0], r[1], r[2], r[3]);
      if (t0 + tl < T) {
        Dims dd{rp.L, 0, NQ, NKV, D, 0, 0, 0.f};
        gfloat* page = page_at(rp.page_table, pos / kPage);
        const int slot = pos % kPage;
        gstore4(page + page_offset(dd, rp.layer, 0, g, slot) + d0, k);
        gstore4(page + page_offset(dd, rp.layer, 1, g, slot) + d0, v);
      }
    }
    vs[d0][tl] = v.x;
    vs[d0 + 1][tl] = v.y;
    vs[d0 + 2][tl] = v.z;
    vs[d0 + 3][tl] = v.w;
    if (t0 + tl < T) {
      const float kk[4] = {k.x, k.y, k.z, k.w};
      __bf16 h4[4], l4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h4[e] = (__bf16)kk[e];
        l4[e] = (__bf16)(kk[e] - (float)h4[e]);
      }
      const size_t o = ((size_t)g * T + t0 + tl) * D + d0;
      *reinterpret_cast<uint2*>(kh + o) = __builtin_bit_cast(uint2, h4);
      *reinterpret_cast<uint2*>(kl + o) = __builtin_bit_cast(uint2, l4);
    }
  }
  __syncthreads();
  // V^T: thread -> column d, 4 consecutive tokens
#pragma unroll
  for (int i = 0; i < TT * D / 4 / 256; ++i) {
    const int c = threadIdx.x + 256 * i, d = c / (TT / 4), tq = 4 * (c % (TT / 4));
    __bf16 h4[4], l4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = vs[d][tq + e];
      h4[e] = (__bf16)v;
      l4[e] = (__bf16)(v - (float)h4[e]);
    }
    // key quad qi of its 32-key group goes to slot 8 qi (qi < 4) or 8 (qi - 4) + 4
    const int qi = (tq % 32) / 4;
    const size_t o = ((size_t)g * D + d) * Tp + t0 + (tq - tq % 32) + (qi < 4 ? 8 * qi : 8 * (qi - 4) + 4);
    *reinterpret_cast<uint2*>(vth + o) = __builtin_bit_cast(uint2, h4);
    *reinterpret_cast<uint2*>(vtl + o) = __builtin_bit_cast(uint2, l4);
  }
}

namespace fa {
constexpr int D = 128;
constexpr int QT = 64;          // query positions per block
constexpr int KT = 32;          // keys per tile
// LDS layouts without bank conflicts on gfx950 (SQ_LDS_BANK_CONFLICT, 16
// bytes per lane from 16 rows): K rows padded to 144 bf16 (288 bytes; 272
// conflicts), V^T rows of 32 bf16 unpadded with chunk c of row r at
// c ^ ((r / 2) % 4) (80-byte padded rows conflict)
constexpr int KP = D + 16;      // bf16 pitch of a K row in LDS
constexpr int VP = KT;          // bf16 pitch of a V^T row in LDS (chunks swizzled)
__device__ __forceinline__ int vt_sw(int d, int chunk) { return d * VP + 8 * (chunk ^ ((d >> 1) & 3)); }
constexpr int KB = KT / 16;     // 16-key blocks per tile
constexpr int KH = KT / 32;     // 32-key groups per tile
}  // namespace fa
// starting exponent base of the online softmax: finite, so that exp2 of a
// masked score (-inf) minus the base is 0, and below any reachable score
constexpr float kFaFloor = -1e30f;

// GROUP query heads share each KV head; QS query blocks of 16 per wave (GROUP
// x QS "virtual heads" v: head g GROUP + v % GROUP, queries 16 (w QS + v / GROUP)
// + [0, 16) of the block). With one query head per KV head, two query blocks
// per wave let every K/V fragment read from LDS feed twice the MFMAs.
template <int GROUP, int QS, int ONEQ>
__global__ __launch_bounds__(256, 2) void attn_prefill_mfma_kernel(const float* __restrict__ qkv, int T, int ld,
                                                                 const uint16_t* __restrict__ khs,
                                                                 const uint16_t* __restrict__ kls,
                                                                 const uint16_t* __restrict__ vths,
                                                                 const uint16_t* __restrict__ vtls, int Tp,
                                                                 float* __restrict__ out, int ldo, float qscale,
                                                                 uint16_t* __restrict__ ohi,
                                                                 uint16_t* __restrict__ olo, int causal,
                                                                 float* __restrict__ part, QkRope rp) {
  using namespace fa;
  // ONEQ: the block takes one query head of the KV head's group (blockIdx.y
  // over the query heads): twice the blocks for a short prompt, each with
  // half the work per K/V tile
  constexpr int GH = ONEQ ? 1 : GROUP;              // query heads per block
  constexpr int VH = GH * QS, QTB = 64 * QS;  // virtual heads per wave, queries per block
  // two tile buffers: the next tile's global loads are in flight while the
  // current one is multiplied, one barrier per tile
  __shared__ __bf16 Kh[2][KT * KP], Kl[2][KT * KP];
  __shared__ __bf16 Vh[2][D * VP], Vl[2][D * VP];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int c16 = lane % 16, gq = lane / 16;
  // Workgroup i runs on XCD i % 8. With a multiple of 8 KV heads and long
  // prompts, head g goes to XCD g % 8, so the blocks sharing an XCD (and its
  // L2) sweep the same K/V tiles at about the same time instead of every L2
  // holding tiles of every head (at T = 8192 the prefill went from 54.3 to
  // 44.8 ms; at T = 1024, where all heads' K/V nearly fit, it measured 1%
  // slower, hence the 32-tile threshold).
  int hy = blockIdx.y, qb = blockIdx.x;
  if (gridDim.y % 8 == 0 && gridDim.x >= 32) {
    // (with ONEQ the query heads of KV head x stay on XCD x)
    const int lin = blockIdx.x + blockIdx.y * gridDim.x, j = lin / 8, x = lin % 8, t = j / gridDim.x;
    hy = ONEQ ? GROUP * (x + 8 * (t / GROUP)) + t % GROUP : x + 8 * t;
    qb = j % gridDim.x;
  }
  const int g = ONEQ ? hy / GROUP : hy;  // KV head
  // query head of virtual head v
  auto qhead = [&](int v) __attribute__((always_inline)) { return ONEQ ? hy : g * GROUP + v % GROUP; };
  // heavier (later) query tiles first
  const int q0 = (gridDim.x - 1 - qb) * QTB;
  int qpv[VH];  // this lane's query position per virtual head
#pragma unroll
  for (int v = 0; v < VH; ++v) qpv[v] = q0 + 16 * (w * QS + v / GH) + c16;

  // Q^T operands (B of S^T = K Q^T): lane supplies Q[query c16][32 s + 8 gq + i]
  // (with rp.norm: the Q-RMSNorm and RoPE of each query first; the lane's
  // columns 32 st + 8 gq + i and their rotate-half partners (st +- 2) are
  // its own, and the 4 lanes of a query share its sum of squares)
  bf16x8_t qh[VH][4], ql[VH][4];
#pragma unroll
  for (int hh = 0; hh < VH; ++hh) {
    const int qrow = min(qpv[hh], T - 1);
    const float* qsrc = qkv + (size_t)qrow * ld + (size_t)qhead(hh) * D + 8 * gq;
    float v[4][8];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float4 a = *reinterpret_cast<const float4*>(qsrc + 32 * st);
      const float4 b = *reinterpret_cast<const float4*>(qsrc + 32 * st + 4);
      v[st][0] = a.x, v[st][1] = a.y, v[st][2] = a.z, v[st][3] = a.w;
      v[st][4] = b.x, v[st][5] = b.y, v[st][6] = b.z, v[st][7] = b.w;
    }
    if (rp.norm) {
      float ss = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(v[st][i], v[st][i], ss);
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      const float inv = 1.f / sqrtf(ss / (float)D + rp.eps);
      float x[4][8];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[st][i] = v[st][i] * inv * rp.q_norm[32 * st + 8 * gq + i];
      const size_t rb = (size_t)(rp.pos0 + qrow) * (D / 2) + 8 * gq;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float c = rp.rcos[rb + 32 * st + i], sn = rp.rsin[rb + 32 * st + i];
          v[st][i] = x[st][i] * c - x[st + 2][i] * sn;
          v[st + 2][i] = x[st + 2][i] * c + x[st][i] * sn;
        }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = v[st][i] * qscale;
        const __bf16 h = (__bf16)x;
        qh[hh][st][i] = h;
        ql[hh][st][i] = (__bf16)(x - (float)h);
      }
    }
  }

  float m[VH], lsum[VH];
  f32x4_t acc[VH][D / 16];
#pragma unroll
  for (int hh = 0; hh < VH; ++hh) {
    m[hh] = kFaFloor;
    lsum[hh] = 0.f;
#pragma unroll
    for (int b = 0; b < D / 16; ++b) acc[hh][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kh_g = khs + (size_t)g * T * D;
  const uint16_t* kl_g = kls + (size_t)g * T * D;
  const uint16_t* vh_g = vths + (size_t)g * D * Tp;
  const uint16_t* vl_g = vtls + (size_t)g * D * Tp;
  // causal: keys up to the block's last query; otherwise every key. With
  // gridDim.z = S > 1 the block's key tiles split into S contiguous ranges,
  // range blockIdx.z here; its unnormalised partial goes to `part`.
  const int last_key = causal ? min(T, q0 + QTB) - 1 : T - 1;
  const int S = gridDim.z, ntile = last_key / KT + 1, per = (ntile + S - 1) / S;
  const int kt_end = min(ntile, ((int)blockIdx.z + 1) * per);
  // copies of the converted tiles: K rows of 16-byte chunks (key c / 16,
  // columns 8 (c % 16)), V^T rows (column d = c / 4, keys 8 (c % 4)); thread
  // t moves chunks c = t and t + 256 of each of the four arrays
  static_assert(KT * D / 8 == 512, "two chunks per thread and array");
  const int kc0 = threadIdx.x / (D / 8), kc1 = kc0 + 256 / (D / 8), kd = 8 * (threadIdx.x % (D / 8));
  const int vd0 = threadIdx.x / (KT / 8), vd1 = vd0 + 256 / (KT / 8), vk = 8 * (threadIdx.x % (KT / 8));
  uint4 rkh0, rkh1, rkl0, rkl1, rvh0, rvh1, rvl0, rvl1;
#define QDEC_FA_LOAD(k0)                                                    \
  {                                                                         \
    const size_t o0 = (size_t)min((k0) + kc0, T - 1) * D + kd;              \
    const size_t o1 = (size_t)min((k0) + kc1, T - 1) * D + kd;              \
    rkh0 = *reinterpret_cast<const uint4*>(kh_g + o0);                      \
    rkh1 = *reinterpret_cast<const uint4*>(kh_g + o1);                      \
    rkl0 = *reinterpret_cast<const uint4*>(kl_g + o0);                      \
    rkl1 = *reinterpret_cast<const uint4*>(kl_g + o1);                      \
    rvh0 = *reinterpret_cast<const uint4*>(vh_g + (size_t)vd0 * Tp + (k0) + vk); \
    rvh1 = *reinterpret_cast<const uint4*>(vh_g + (size_t)vd1 * Tp + (k0) + vk); \
    rvl0 = *reinterpret_cast<const uint4*>(vl_g + (size_t)vd0 * Tp + (k0) + vk); \
    rvl1 = *reinterpret_cast<const uint4*>(vl_g + (size_t)vd1 * Tp + (k0) + vk); \
  }
#define QDEC_FA_STORE(b)                                           \
  {                                                                \
    *reinterpret_cast<uint4*>(&Kh[b][kc0 * KP + kd]) = rkh0;       \
    *reinterpret_cast<uint4*>(&Kh[b][kc1 * KP + kd]) = rkh1;       \
    *reinterpret_cast<uint4*>(&Kl[b][kc0 * KP + kd]) = rkl0;       \
    *reinterpret_cast<uint4*>(&Kl[b][kc1 * KP + kd]) = rkl1;       \
    *reinterpret_cast<uint4*>(&Vh[b][vt_sw(vd0, vk / 8)]) = rvh0;  \
    *reinterpret_cast<uint4*>(&Vh[b][vt_sw(vd1, vk / 8)]) = rvh1;  \
    *reinterpret_cast<uint4*>(&Vl[b][vt_sw(vd0, vk / 8)]) = rvl0;  \
    *reinterpret_cast<uint4*>(&Vl[b][vt_sw(vd1, vk / 8)]) = rvl1;  \
  }
  const int kbeg = blockIdx.z * per * KT, kend = kt_end * KT;
  if (kbeg < kend) {
    QDEC_FA_LOAD(kbeg)
    QDEC_FA_STORE(0)
  }
  __syncthreads();
  for (int k0 = kbeg, buf = 0; k0 < kend; k0 += KT, buf ^= 1) {
    // the next tile (the last iteration reloads its own: the store below
    // then fills a buffer nobody reads)
    const int kn = k0 + KT < kend ? k0 + KT : k0;
    QDEC_FA_LOAD(kn)

    // S^T tile: KB key blocks of 16 x this wave's 16 queries, per head
    f32x4_t sc[VH][KB];
#pragma unroll
    for (int hh = 0; hh < VH; ++hh)
#pragma unroll
      for (int j = 0; j < KB; ++j) sc[hh][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int off = (16 * j + c16) * KP + 32 * st + 8 * gq;
        const bf16x8_t kh = *reinterpret_cast<const bf16x8_t*>(&Kh[buf][off]);
        const bf16x8_t kl = *reinterpret_cast<const bf16x8_t*>(&Kl[buf][off]);
#pragma unroll
        for (int hh = 0; hh < VH; ++hh) {
          sc[hh][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[hh][st], sc[hh][j], 0, 0, 0);
          sc[hh][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[hh][st], sc[hh][j], 0, 0, 0);
          sc[hh][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[hh][st], sc[hh][j], 0, 0, 0);
        }
      }

    // online softmax per head; P^T operands per 32-key group. Only tiles
    // that reach past this wave's first query (or past T) need the mask.
    const bool full = k0 + KT <= T && (!causal || k0 + KT - 1 <= q0 + 16 * w * QS);
    float mx[VH];
#pragma unroll
    for (int hh = 0; hh < VH; ++hh) {
      if (!full) {
        const int qlim = causal ? qpv[hh] : T - 1;  // this lane's last visible key
#pragma unroll
        for (int j = 0; j < KB; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + 16 * j + 4 * gq + e;
            if (key > qlim || key >= T) sc[hh][j][e] = -INFINITY;
          }
      }
      float v = m[hh];
#pragma unroll
      for (int j = 0; j < KB; ++j) v = fmaxf(v, fmaxf(fmaxf(sc[hh][j][0], sc[hh][j][1]), fmaxf(sc[hh][j][2], sc[hh][j][3])));
      v = fmaxf(v, __shfl_xor(v, 16, kWave));
      mx[hh] = fmaxf(v, __shfl_xor(v, 32, kWave));
    }
    // The exponent base m moves only when a score passes it by more than 8
    // (a factor of 256 in the probabilities): the normalised result is the
    // same for any base, and most tiles then skip rescaling the output
    // accumulators (the branch is taken by the whole wave or not at all). Key
    // 0 is visible to every query, so the first tile sets the base; m starts
    // at a finite floor, so a masked score (-inf) always gives p = 0.
    bool move = false;
#pragma unroll
    for (int hh = 0; hh < VH; ++hh) move = move || mx[hh] > m[hh] + 8.f;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
      for (int hh = 0; hh < VH; ++hh) {
        const bool mv = mx[hh] > m[hh] + 8.f;
        const float alpha = mv ? __builtin_amdgcn_exp2f(m[hh] - mx[hh]) : 1.f;
        lsum[hh] *= alpha;
#pragma unroll
        for (int b = 0; b < D / 16; ++b) acc[hh][b] *= alpha;
        m[hh] = mv ? mx[hh] : m[hh];
      }
    }
    bf16x8_t ph[VH][KH], pl[VH][KH];
#pragma unroll
    for (int hh = 0; hh < VH; ++hh) {
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(sc[hh][j][e] - m[hh]);
          ps += p;
          const __bf16 h = (__bf16)p;
          ph[hh][j / 2][4 * (j % 2) + e] = h;
          pl[hh][j / 2][4 * (j % 2) + e] = (__bf16)(p - (float)h);
        }
      ps += __shfl_xor(ps, 16, kWave);
      ps += __shfl_xor(ps, 32, kWave);
      lsum[hh] += ps;
    }

    // O^T += V^T P^T: d block b, 32-key group c
#pragma unroll
    for (int b = 0; b < D / 16; ++b)
#pragma unroll
      for (int c = 0; c < KH; ++c) {
        // keys 4 gq + e and 16 + 4 gq + e of the group sit together at 8 gq
        const int off = vt_sw(16 * b + c16, 4 * c + gq);
        const bf16x8_t vh = *reinterpret_cast<const bf16x8_t*>(&Vh[buf][off]);
        const bf16x8_t vl = *reinterpret_cast<const bf16x8_t*>(&Vl[buf][off]);
#pragma unroll
        for (int hh = 0; hh < VH; ++hh) {
          acc[hh][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh, ph[hh][c], acc[hh][b], 0, 0, 0);
          acc[hh][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl, ph[hh][c], acc[hh][b], 0, 0, 0);
          acc[hh][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh, pl[hh][c], acc[hh][b], 0, 0, 0);
        }
      }
    // the other buffer was last read before the previous barrier
    QDEC_FA_STORE(buf ^ 1)
    __syncthreads();
  }
#undef QDEC_FA_LOAD
#undef QDEC_FA_STORE

  if (S > 1) {
    // partial of split z: o (unnormalised), the exponent base m and the sum l
    // per (query, head), records of D + 4 floats (16-byte aligned) at
    // part[((z T + q) NQ + h) (D + 4)] (NQ = ldo / D)
    const int nq = ldo / D;
#pragma unroll
    for (int hh = 0; hh < VH; ++hh) {
      if (qpv[hh] < T) {
        float* pp = part + (((size_t)blockIdx.z * T + qpv[hh]) * nq + qhead(hh)) * (D + 4);
#pragma unroll
        for (int b = 0; b < D / 16; ++b)
          *reinterpret_cast<float4*>(pp + 16 * b + 4 * gq) =
              make_float4(acc[hh][b][0], acc[hh][b][1], acc[hh][b][2], acc[hh][b][3]);
        if (gq == 0) {
          pp[D] = lsum[hh] > 0.f ? m[hh] : -INFINITY;  // no visible key: the merge skips it
          pp[D + 1] = lsum[hh];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int hh = 0; hh < VH; ++hh) {
    if (qpv[hh] < T) {
      const float il = 1.f / lsum[hh];
      const size_t o = (size_t)qpv[hh] * ldo + (size_t)qhead(hh) * D + 4 * gq;
#pragma unroll
      for (int b = 0; b < D / 16; ++b) {
        const float v[4] = {acc[hh][b][0] * il, acc[hh][b][1] * il, acc[hh][b][2] * il, acc[hh][b][3] * il};
        if (ohi) {
          // the O projection's operand directly: bf16 hi = bf16(v), lo = bf16(v - hi)
          // of the rounded fp32 v (no contraction into the product above)
#pragma clang fp contract(off)
          uint16_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[e] = f32_to_bf16_rne(v[e]);
            l[e] = f32_to_bf16_rne(v[e] - bf16_to_f32(h[e]));
          }
          *reinterpret_cast<uint2*>(ohi + o + 16 * b) = make_uint2(h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16));
          *reinterpret_cast<uint2*>(olo + o + 16 * b) = make_uint2(l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16));
        } else {
          *reinterpret_cast<float4*>(out + o + 16 * b) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

// Merge of S key-range partials of the prefill attention: for query q and
// head h, with bases m_z and sums l_z, o = sum_z 2^(m_z - M) o_z /
// sum_z 2^(m_z - M) l_z, M = max_z m_z, in split order; written as fp32
// (out) or as the O projection's bf16 hi / lo operand. A split that saw no
// key has m = -inf, l = 0.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part, int S, int T, int nq,
                                                         float* __restrict__ out, uint16_t* __restrict__ ohi,
                                                         uint16_t* __restrict__ olo) {
  // 8 (query, head) records per block, 32 threads per record, 4 dimensions
  // per thread
  constexpr int D = fa::D;
  const int rec = blockIdx.x * 8 + threadIdx.x / 32, d = 4 * (threadIdx.x % 32);
  if (rec >= T * nq) return;
  const size_t zs = (size_t)T * nq * (D + 4);  // one split's records
  const float* p0 = part + (size_t)rec * (D + 4);
  float mx = -INFINITY;
  for (int z = 0; z < S; ++z) mx = fmaxf(mx, p0[z * zs + D]);
  float o[4] = {0.f, 0.f, 0.f, 0.f}, l = 0.f;
  for (int z = 0; z < S; ++z) {
    const float* pp = p0 + z * zs;
    const float mz = pp[D];
    const float wz = mz == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mz - mx);
    const float4 v = *reinterpret_cast<const float4*>(pp + d);
    o[0] = fmaf(wz, v.x, o[0]);
    o[1] = fmaf(wz, v.y, o[1]);
    o[2] = fmaf(wz, v.z, o[2]);
    o[3] = fmaf(wz, v.w, o[3]);
    l = fmaf(wz, pp[D + 1], l);
  }
  const size_t idx = (size_t)rec * D + d;
  const float v[4] = {o[0] / l, o[1] / l, o[2] / l, o[3] / l};
  if (ohi) {
#pragma clang fp contract(off)
    uint16_t h[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = f32_to_bf16_rne(v[e]);
      lo[e] = f32_to_bf16_rne(v[e] - bf16_to_f32(h[e]));
    }
    *reinterpret_cast<uint2*>(ohi + idx) = make_uint2(h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16));
    *reinterpret_cast<uint2*>(olo + idx) = make_uint2(lo[0] | ((unsigned)lo[1] << 16), lo[2] | ((unsigned)lo[3] << 16));
  } else {
    *reinterpret_cast<float4*>(out + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// ------------------------------------------------ prefill activations / GEMM
// Activations are fp32; the bf16 MFMA consumes them as hi + lo bf16 pairs
// (hi = bf16(v), lo = bf16(v - hi)), two MFMAs per tile, which keeps about 16
// mantissa bits of every product against the exact bf16 weights.

__global__ __launch_bounds__(256) void rms_split_kernel(const float* __restrict__ X, int K,
                                                         const float* __restrict__ gain, float eps,
                                                         uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  __shared__ float red[8];
  const int t = blockIdx.x;
  const float* x = X + (size_t)t * K;
  float inv = 1.f;
  if (gain) {
    float ss = 0.f;
    for (int i = threadIdx.x; i < K; i += blockDim.x) ss = fmaf(x[i], x[i], ss);
    ss = block_sum(ss, red);
    inv = 1.f / sqrtf(ss / (float)K + eps);
  }
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const float v = gain ? x[i] * inv * gain[i] : x[i];
    const uint16_t h = f32_to_bf16_rne(v);
    hi[(size_t)t * K + i] = h;
    lo[(size_t)t * K + i] = f32_to_bf16_rne(v - bf16_to_f32(h));
  }
}

// The same for rows of K % 4 == 0, K <= 4 * 256 * R: each thread keeps its
// float4 chunks c = tid + 256 r in registers, so the row is read once, and
// writes 8-byte hi / lo groups.
template <int R>
__global__ __launch_bounds__(256) void rms_split_vec_kernel(const float* __restrict__ X, int K,
                                                             const float* __restrict__ gain, float eps,
                                                             uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  __shared__ float red[8];
  const int t = blockIdx.x, nc = K / 4;
  const float4* x = reinterpret_cast<const float4*>(X + (size_t)t * K);
  float4 v[R];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = threadIdx.x + 256 * r;
    v[r] = c < nc ? x[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss = fmaf(v[r].x, v[r].x, fmaf(v[r].y, v[r].y, fmaf(v[r].z, v[r].z, fmaf(v[r].w, v[r].w, ss))));
  }
  float inv = 1.f;
  if (gain) inv = 1.f / sqrtf(block_sum(ss, red) / (float)K + eps);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = threadIdx.x + 256 * r;
    if (c < nc) {
      float e[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
      if (gain) {
        const float4 g = reinterpret_cast<const float4*>(gain)[c];
        e[0] = e[0] * inv * g.x;
        e[1] = e[1] * inv * g.y;
        e[2] = e[2] * inv * g.z;
        e[3] = e[3] * inv * g.w;
      }
      uint16_t h[4], l[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = f32_to_bf16_rne(e[k]);
        l[k] = f32_to_bf16_rne(e[k] - bf16_to_f32(h[k]));
      }
      const size_t o = (size_t)t * K + 4 * c;
      *reinterpret_cast<uint2*>(hi + o) = make_uint2(h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16));
      *reinterpret_cast<uint2*>(lo + o) = make_uint2(l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16));
    }
  }
}

// LayerNorm of each row (mean and population variance over K, gain and bias)
// written as the next GEMM's bf16 hi/lo operand. Block = one row.
__global__ __launch_bounds__(256) void ln_split_kernel(const float* __restrict__ X, int K,
                                                        const float* __restrict__ gain, const float* __restrict__ bias,
                                                        float eps, uint16_t* __restrict__ hi,
                                                        uint16_t* __restrict__ lo, int ldo) {
  __shared__ float red[8];
  const int t = blockIdx.x;
  const float* x = X + (size_t)t * K;
  float s = 0.f;
  for (int i = threadIdx.x; i < K; i += blockDim.x) s += x[i];
  const float mean = block_sum(s, red) / (float)K;
  float ss = 0.f;
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const float c = x[i] - mean;
    ss = fmaf(c, c, ss);
  }
  const float inv = 1.f / sqrtf(block_sum(ss, red) / (float)K + eps);
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const float v = (x[i] - mean) * inv * gain[i] + bias[i];
    const uint16_t h = f32_to_bf16_rne(v);
    hi[(size_t)t * ldo + i] = h;
    lo[(size_t)t * ldo + i] = f32_to_bf16_rne(v - bf16_to_f32(h));
  }
  for (int i = K + threadIdx.x; i < ldo; i += blockDim.x) {
    hi[(size_t)t * ldo + i] = 0;
    lo[(size_t)t * ldo + i] = 0;
  }
}

__global__ __launch_bounds__(256) void rms_apply_kernel(const float* __restrict__ X, int K,
                                                         const float* __restrict__ gain, float eps,
                                                         float* __restrict__ out) {
  __shared__ float red[8];
  const int t = blockIdx.x;
  const float* x = X + (size_t)t * K;
  float inv = 1.f;
  if (gain) {
    float ss = 0.f;
    for (int i = threadIdx.x; i < K; i += blockDim.x) ss = fmaf(x[i], x[i], ss);
    ss = block_sum(ss, red);
    inv = 1.f / sqrtf(ss / (float)K + eps);
  }
  for (int i = threadIdx.x; i < K; i += blockDim.x) out[(size_t)t * K + i] = gain ? x[i] * inv * gain[i] : x[i];
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// C[M, N] (+)= (Ahi + Alo)[M, K] . W[N, K]^T with bf16 MFMA 16x16x32.
// Block tile 64 x 64, 4 waves in 2 x 2, each wave 2 x 2 MFMA tiles.
// MFMA operand layout (16x16x32): lane l supplies A[l % 16][8 (l / 16) + 0..7]
// and B[8 (l / 16) + 0..7][l % 16]; it receives D[4 (l / 16) + 0..3][l % 16].
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16x2_kernel(const uint16_t* __restrict__ Ahi,
                                                           const uint16_t* __restrict__ Alo, int M, int K,
                                                           const uint16_t* __restrict__ W, int N,
                                                           float* __restrict__ C, int ldc,
                                                           const float* __restrict__ bias) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int m0 = blockIdx.y * 64 + (wave / 2) * 32;
  const int n0 = blockIdx.x * 64 + (wave % 2) * 32;
  const int r = lane % 16, kq = (lane / 16) * 8;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // rows and columns past the edge repeat the last one: an MFMA output
  // element depends only on its own A row and W row, and those are never
  // stored (a select against zero here put the operands in scratch)
  for (int k = 0; k < K; k += 32) {
    uint4 ah[2], al[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = min(m0 + i * 16 + r, M - 1);
      ah[i] = *reinterpret_cast<const uint4*>(Ahi + (size_t)row * K + k + kq);
      al[i] = *reinterpret_cast<const uint4*>(Alo + (size_t)row * K + k + kq);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = min(n0 + j * 16 + r, N - 1);
      b[j] = *reinterpret_cast<const uint4*>(W + (size_t)col * K + k + kq);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah[i]),
                                                            __builtin_bit_cast(bf16x8_t, b[j]), acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al[i]),
                                                            __builtin_bit_cast(bf16x8_t, b[j]), acc[i][j], 0, 0, 0);
      }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + j * 16 + (lane % 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + i * 16 + 4 * (lane / 16) + e;
        float v = acc[i][j][e];
        if (EPI == EPI_SWIGLU) {
          const float u = __shfl_xor(v, 8, kWave);
          if ((lane % 16) < kGuGroup && row < M && col < N)
            C[(size_t)row * ldc + (col / 16) * kGuGroup + (lane % 8)] = silu_mul(v, u);
        } else if (row < M && col < N) {
          if (bias) v += bias[col];
          if (EPI == EPI_RESID)
            C[(size_t)row * ldc + col] += v;
          else if (EPI == EPI_RELU)
            C[(size_t)row * ldc + col] = fmaxf(v, 0.f);
          else
            C[(size_t)row * ldc + col] = v;
        }
      }
    }
}

// Small-M GEMM with fused prologue and epilogue, for up to 64 activation rows
// (batched decode, short prompts): C[M, N] = op(A)[M, K] . W[N, K]^T.
// op(A) is A itself or, with NORM, the RMS-normalised rows A * inv * gain,
// inv = 1 / sqrt(sum(ssq partials of the row) / K + eps); with bf16 weights
// the fp32 values are split into bf16 hi + lo in registers for the MFMAs,
// with fp32 weights (fp32 models, the dequantized copies of Q8_0 models)
// they go unsplit to the fp32 MFMA: a lane's 8 consecutive k of its A row and
// of its W row feed 8 16x16x4 products, product e taking element e, so each
// covers k = e, 8 + e, 16 + e, 24 + e of the 32-wide step. Workgroup =
// (16 NT output columns, K chunk of KC), 4 waves splitting the chunk; the
// waves' sums meet in LDS. With several chunks, each workgroup stores its
// partial tile, and the last to arrive at the column tile (arrival counter,
// reset by that workgroup) adds all partials in chunk order, so the result
// does not depend on scheduling. Epilogues:
//   STORE   C = v
//   RESID   C += v, and ssq_out[tile][row] = sum over the tile's columns of
//           the new C^2 (the next NORM prologue's partials)
//   SWIGLU  columns come as 8 gate then 8 up rows per group of 16; output j
//           of group q is silu(gate) * up at C[row][8q + j]
//   HEAD    C = v when C is set; keys[row] = max(keys[row], argmax key)
template <int MT, int NT, bool NORM, typename WT>
struct RowsStep {
  static constexpr bool F32 = std::is_same<WT, float>::value;
  static constexpr int WB = F32 ? 2 : 1;  // 16-byte loads per lane of a W row's 8 k
  uint4 b[NT][WB];
  float4 a[MT][2];
  float4 gv[2];
  __device__ __forceinline__ void load(const WT* const* wrow, const float* const* arow, const float* gk, int k) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int h = 0; h < WB; ++h) b[j][h] = *reinterpret_cast<const uint4*>(wrow[j] + k + 4 * h);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      a[i][0] = *reinterpret_cast<const float4*>(arow[i] + k);
      a[i][1] = *reinterpret_cast<const float4*>(arow[i] + k + 4);
    }
    if (NORM) {
      gv[0] = *reinterpret_cast<const float4*>(gk + k);
      gv[1] = *reinterpret_cast<const float4*>(gk + k + 4);
    }
  }
  __device__ __forceinline__ void mma(f32x4_t (&acc)[MT][NT], const float* inv) const {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float v[8] = {a[i][0].x, a[i][0].y, a[i][0].z, a[i][0].w, a[i][1].x, a[i][1].y, a[i][1].z, a[i][1].w};
      if (NORM) {
        const float g8[8] = {gv[0].x, gv[0].y, gv[0].z, gv[0].w, gv[1].x, gv[1].y, gv[1].z, gv[1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * inv[i] * g8[e];
      }
      if constexpr (F32) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const float w8[8] = {__uint_as_float(b[j][0].x), __uint_as_float(b[j][0].y), __uint_as_float(b[j][0].z),
                               __uint_as_float(b[j][0].w), __uint_as_float(b[j][1].x), __uint_as_float(b[j][1].y),
                               __uint_as_float(b[j][1].z), __uint_as_float(b[j][1].w)};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[e], w8[e], acc[i][j], 0, 0, 0);
        }
        continue;
      }
      bf16x8_t hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = (__bf16)v[e];
        lo[e] = (__bf16)(v[e] - (float)hi[e]);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, __builtin_bit_cast(bf16x8_t, b[j][0]), acc[i][j], 0,
                                                            0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, __builtin_bit_cast(bf16x8_t, b[j][0]), acc[i][j], 0,
                                                            0, 0);
      }
    }
  }
};

constexpr unsigned long long kRowsWaitTicks = 200000000ull;  // about 0.1 s of s_memtime

template <int MT, int NT, int EPI, bool NORM, typename WT>
__global__ __launch_bounds__(256) void gemm_rows_kernel(RowsGemm g) {
  constexpr int U = 4;                 // k-steps of loads in flight per wave
  constexpr int S = MT * NT * 4;       // accumulator floats per lane
  constexpr int TR = MT * 16, TC = NT * 16;
  __shared__ float red[4][S][kWave];
  __shared__ float tv[TR][TC + 1];
  __shared__ int s_last;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int tile = blockIdx.x, c = blockIdx.y, nkc = gridDim.y;
  const int n0 = tile * TC, m0 = blockIdx.z * TR;  // output tile: rows m0 + [0, TR), columns n0 + [0, TC)
  const int M = g.M, K = g.K;
  const int kw = g.KC / 4;
  const int kb = c * g.KC + wave * kw, ke = min(K, kb + kw);
  const int r = lane % 16, kq = (lane / 16) * 8;

  const WT* wrow[NT];
  const float* arow[MT];
  float inv[MT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wrow[j] = (const WT*)g.W + (size_t)(n0 + j * 16 + r) * K + kq;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    // rows past M repeat row M - 1: an MFMA output row depends only on its
    // own A row, and those rows are never stored
    const int row = min(m0 + i * 16 + r, M - 1);
    arow[i] = g.A + (size_t)row * g.lda + kq;
    inv[i] = 1.f;
    if (NORM) {
      // the 4 lanes of a row split the partials, then meet by butterfly
      // (every lane of the row ends with the same sum)
      float ss = 0.f;
#pragma unroll 8
      for (int t = lane / 16; t < g.nss; t += 4) ss += g.ssq[(size_t)t * M + row];
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      inv[i] = 1.f / sqrtf(ss / (float)K + g.eps);
    }
  }
  const float* gk = NORM ? g.gain + kq : nullptr;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int k = kb;
  for (; k + 32 * U <= ke; k += 32 * U) {
    RowsStep<MT, NT, NORM, WT> st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) st[u].load(wrow, arow, gk, k + 32 * u);
    // every load of the batch ahead of the first multiply
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) st[u].mma(acc, inv);
  }
  for (; k < ke; k += 32) {
    RowsStep<MT, NT, NORM, WT> st;
    st.load(wrow, arow, gk, k);
    st.mma(acc, inv);
  }

  // the 4 waves' sums, in wave order; thread (wave w, lane l) then owns the
  // slots s = 4 q + w, s = 4 (i NT + j) + e <-> row 16 i + 4 (l / 16) + e,
  // column 16 j + l % 16 of the tile
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][(i * NT + j) * 4 + e][lane] = acc[i][j][e];
  __syncthreads();
  float v[MT * NT];
#pragma unroll
  for (int q = 0; q < MT * NT; ++q) {
    const int sl = 4 * q + wave;
    v[q] = ((red[0][sl][lane] + red[1][sl][lane]) + red[2][sl][lane]) + red[3][sl][lane];
  }

  if (nkc > 1) {
    // Partials travel as 8-byte words (tag of this launch, value) written and
    // read at device scope, so a word is either absent or whole, and no cache
    // flush is needed. The workgroup that brings the tile's counter to nkc
    // has seen every other workgroup's stores complete before their
    // increments; it still checks each tag, waiting (bounded) for a word
    // that is not yet visible.
    const int ot = blockIdx.z * gridDim.x + tile;  // output tile index
    unsigned long long* pt = g.P + (size_t)ot * S * kWave;
    const size_t cstride = (size_t)gridDim.x * gridDim.z * S * kWave;
    const unsigned long long tag = (unsigned long long)g.tag << 32;
#pragma unroll
    for (int q = 0; q < MT * NT; ++q)
      __hip_atomic_store(pt + c * cstride + (4 * q + wave) * kWave + lane, tag | __float_as_uint(v[q]),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // stores acknowledged before the barrier, so before the increment
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(g.cnt + ot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (unsigned)(nkc - 1);
    __syncthreads();
    if (!s_last) return;
    // all chunks' words requested at once, 8 chunks per round (addresses
    // clamped to the last chunk, surplus words ignored), then summed in
    // chunk order
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    bool late = false;
    float t[MT * NT];
#pragma unroll
    for (int q = 0; q < MT * NT; ++q) t[q] = 0.f;
    for (int cb = 0; cb < nkc; cb += 8) {
      unsigned long long w[MT * NT][8];
#pragma unroll
      for (int q = 0; q < MT * NT; ++q)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          w[q][u] = __hip_atomic_load(pt + min(cb + u, nkc - 1) * cstride + (4 * q + wave) * kWave + lane,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int q = 0; q < MT * NT; ++q)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int cc = cb + u;
          if (cc < nkc) {
            if (cc == c) {
              t[q] += v[q];
            } else {
              while ((w[q][u] >> 32) != g.tag && !late) {
                late = __builtin_amdgcn_s_memtime() - t0 > kRowsWaitTicks;
                w[q][u] = __hip_atomic_load(pt + cc * cstride + (4 * q + wave) * kWave + lane, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
              }
              t[q] += (w[q][u] >> 32) == g.tag ? __uint_as_float((unsigned)w[q][u]) : __builtin_nanf("");
            }
          }
        }
    }
#pragma unroll
    for (int q = 0; q < MT * NT; ++q) v[q] = t[q];
    if (late) __hip_atomic_store(g.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (threadIdx.x == 0) __hip_atomic_store(g.cnt + ot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int q = 0; q < MT * NT; ++q) {
    const int sl = 4 * q + wave;
    const int e = sl % 4, ij = sl / 4, i = ij / NT, j = ij % NT;
    tv[16 * i + 4 * (lane / 16) + e][16 * j + lane % 16] = v[q];
  }
  __syncthreads();

  if (EPI == EPI_SWIGLU) {
    for (int idx = threadIdx.x; idx < TR * NT * 8; idx += blockDim.x) {
      const int rt = idx / (NT * 8), o = idx % (NT * 8), j = o / 8, e = o % 8;
      if (m0 + rt < M)
        g.C[(size_t)(m0 + rt) * g.ldc + (n0 / 16 + j) * 8 + e] = silu_mul(tv[rt][16 * j + e], tv[rt][16 * j + 8 + e]);
    }
    return;
  }
  if (EPI != EPI_HEAD || g.C) {
    for (int idx = threadIdx.x; idx < TR * TC; idx += blockDim.x) {
      const int rt = idx / TC, ct = idx % TC;
      if (m0 + rt < M) {
        float* dst = g.C + (size_t)(m0 + rt) * g.ldc + n0 + ct;
        if (EPI == EPI_RESID) {
          const float x = *dst + tv[rt][ct];
          *dst = x;
          tv[rt][ct] = x;
        } else {
          *dst = tv[rt][ct];
        }
      }
    }
  }
  if (EPI == EPI_RESID) {
    __syncthreads();
    if (threadIdx.x < TR && m0 + (int)threadIdx.x < M) {
      float ss = 0.f;
      for (int ct = 0; ct < TC; ++ct) ss = fmaf(tv[threadIdx.x][ct], tv[threadIdx.x][ct], ss);
      g.ssq_out[(size_t)tile * M + m0 + threadIdx.x] = ss;
    }
  }
  if (EPI == EPI_HEAD && threadIdx.x < TR && m0 + (int)threadIdx.x < M) {
    unsigned long long best = 0ull;
    for (int ct = 0; ct < TC; ++ct) {
      const unsigned long long kk = argmax_key(tv[threadIdx.x][ct], n0 + ct);
      best = kk > best ? kk : best;
    }
    atomicMax(g.keys + (size_t)(m0 + threadIdx.x) * kKeySlots + tile % kKeySlots, best);
  }
}

// Large-M GEMM (prefill): C[M, N] (+)= (Ahi + Alo)[M, K] . W[N, K]^T with
// 128 x 128 (or 64 x 128) output tiles and K steps of 32 staged in LDS
// (double buffered: the next step's global loads are in flight while the
// current one is multiplied). 4 waves in a 2 x 2 arrangement, each 64 x 64
// (or 32 x 64) = 4 x 4 (or 2 x 4) MFMA tiles of 16 x 16, two MFMAs (hi, lo)
// per tile and step. LDS rows are 64
// bytes with XOR-swizzled 16-byte chunks (tg_sw). Epilogues as in
// gemm_bf16x2_kernel.
namespace tg {
constexpr int BN = 128, BK = 32;
constexpr size_t kTiledWSliceBytes = size_t(3) << 20;  // W bytes per XCD column group
constexpr int P = BK;  // bf16 pitch of an LDS row (chunks XOR-swizzled)
// 16-byte chunk c of LDS row r sits at chunk c ^ ((r / 2) % 4): an MFMA
// operand read (16 rows, one chunk each) is then free of bank conflicts
// without padding, which keeps the double-buffered tiles at 48 KB (three
// workgroups per CU). Measured with the SQ_LDS_BANK_CONFLICT counter on
// gfx950: a 16-byte-per-lane read of 64-byte rows conflicts (about 4 extra
// cycles per read) unpadded, padded to 80 bytes, or swizzled by (r / 4) % 4,
// and is conflict-free swizzled by (r / 2) % 4.
__device__ __forceinline__ int tg_sw(int r, int c) { return r * P + 8 * (c ^ ((r >> 1) & 3)); }
}  // namespace tg

// Split-K of the tiled GEMM (grid z = split): split z covers K steps
// [z kc, (z + 1) kc) / BK and stores its fp32 partial of C to
// P[z][row][col]; splitk_reduce_kernel then sums the splits in order and
// applies the epilogue (the kernel boundary makes every partial visible).
struct TiledSplit {
  float* P;  // splits * M * N floats (null: no split)
  int kc;    // K per split (a multiple of BK)
};

template <int EPI, int MW, int SUBT>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const uint16_t* __restrict__ Ahi,
                                                          const uint16_t* __restrict__ Alo, int M, int K,
                                                          const uint16_t* __restrict__ W, int N,
                                                          float* __restrict__ C, int ldc,
                                                          uint16_t* __restrict__ Zhi,
                                                          uint16_t* __restrict__ Zlo,
                                                          const float* __restrict__ bias, TiledSplit sp) {
  using namespace tg;
  // MW 16-row MFMA tiles per wave along M: 128-row tiles (MW = 4) or
  // 64-row tiles (MW = 2, twice the workgroups for the same shape)
  static_assert(MW == 4 || MW == 2, "128- or 64-row tiles");
  constexpr int TM = 32 * MW;
  // SUB K sub-steps of 32 per LDS buffer and barrier (64-row tiles: 2 where
  // the K range allows, halving the barriers per MFMA)
  constexpr int SUB = MW == 2 ? SUBT : 1;
  constexpr int KS = BK * SUB;  // K per step
  __shared__ uint16_t sAh[2][SUB][TM * P], sAl[2][SUB][TM * P], sW[2][SUB][BN * P];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int c16 = lane % 16, gq = lane / 16;
  const int wm = w / 2, wn = w % 2;
  // Workgroup i runs on XCD i % 8. The tiles are dealt so that each XCD owns
  // one of gc column groups and one of 8 / gc row groups, gc the smallest
  // power of two that keeps its W slice within kTiledWSliceBytes (so the slice
  // stays in the XCD's L2 while the XCD sweeps its row tiles, column fastest).
  // Launch order alone would give every XCD a column slice of every row tile,
  // so all eight L2s would read all of A.
  int tile = blockIdx.x + blockIdx.y * gridDim.x;
  {
    const size_t wbytes = (size_t)N * K * 2;
    int gc = 1;
    while (gc < 8 && (wbytes > (size_t)gc * kTiledWSliceBytes || gridDim.y % (8 / gc) != 0)) gc *= 2;
    if (gridDim.x % gc == 0 && gridDim.y % (8 / gc) == 0) {
      const int x = tile % 8, j = tile / 8;
      const int cw = gridDim.x / gc, rh = gridDim.y / (8 / gc);
      tile = ((x / gc) * rh + j / cw) * gridDim.x + (x % gc) * cw + j % cw;
    }
  }
  const int n0 = (tile % gridDim.x) * BN, m0 = (tile / gridDim.x) * TM;

  // staging: rows of 4 chunks of 16 bytes per matrix; thread t moves chunks
  // t and t + 256 (rows t / 4 and t / 4 + 64, chunk t % 4), the second A
  // chunk only with 128-row tiles
  const int srow = threadIdx.x / 4, skc = threadIdx.x % 4;
  const size_t a0 = (size_t)min(m0 + srow, M - 1) * K + 8 * skc;
  const size_t a1 = (size_t)min(m0 + srow + 64, M - 1) * K + 8 * skc;
  const size_t w0 = (size_t)(n0 + srow) * K + 8 * skc;
  const size_t w1 = (size_t)(n0 + srow + 64) * K + 8 * skc;
  const int l0 = tg_sw(srow, skc), l1 = tg_sw(srow + 64, skc);
  // two register sets (X, Y) of one K step's chunks: with 64-row tiles a
  // step's global loads are issued two steps before its LDS store, so they
  // have two steps of MFMA work to land
  // (named registers per sub-step, not arrays: arrays indexed in a macro's
  // loop went to scratch)
  uint4 rh0X0, rh1X0, rl0X0, rl1X0, rw0X0, rw1X0, rh0Y0, rh1Y0, rl0Y0, rl1Y0, rw0Y0, rw1Y0;
  uint4 rh0X1, rh1X1, rl0X1, rl1X1, rw0X1, rw1X1, rh0Y1, rh1Y1, rl0Y1, rl1Y1, rw0Y1, rw1Y1;
#define QDEC_TG_LD(R, S_, k)                                                  \
  {                                                                           \
    rh0##R##S_ = *reinterpret_cast<const uint4*>(Ahi + a0 + (k) + BK * S_);   \
    rl0##R##S_ = *reinterpret_cast<const uint4*>(Alo + a0 + (k) + BK * S_);   \
    if constexpr (MW == 4) {                                                  \
      rh1##R##S_ = *reinterpret_cast<const uint4*>(Ahi + a1 + (k) + BK * S_); \
      rl1##R##S_ = *reinterpret_cast<const uint4*>(Alo + a1 + (k) + BK * S_); \
    }                                                                         \
    rw0##R##S_ = *reinterpret_cast<const uint4*>(W + w0 + (k) + BK * S_);     \
    rw1##R##S_ = *reinterpret_cast<const uint4*>(W + w1 + (k) + BK * S_);     \
  }
#define QDEC_TG_ST(R, S_, buf)                                                \
  {                                                                           \
    *reinterpret_cast<uint4*>(&sAh[buf][S_][l0]) = rh0##R##S_;                \
    *reinterpret_cast<uint4*>(&sAl[buf][S_][l0]) = rl0##R##S_;                \
    if constexpr (MW == 4) {                                                  \
      *reinterpret_cast<uint4*>(&sAh[buf][S_][l1]) = rh1##R##S_;              \
      *reinterpret_cast<uint4*>(&sAl[buf][S_][l1]) = rl1##R##S_;              \
    }                                                                         \
    *reinterpret_cast<uint4*>(&sW[buf][S_][l0]) = rw0##R##S_;                 \
    *reinterpret_cast<uint4*>(&sW[buf][S_][l1]) = rw1##R##S_;                 \
  }
#define QDEC_TG_LOAD(R, k)               \
  {                                      \
    QDEC_TG_LD(R, 0, k)                  \
    if constexpr (SUB == 2) QDEC_TG_LD(R, 1, k) \
  }
#define QDEC_TG_STORE(R, buf)            \
  {                                      \
    QDEC_TG_ST(R, 0, buf)                \
    if constexpr (SUB == 2) QDEC_TG_ST(R, 1, buf) \
  }
#define QDEC_TG_MMA(buf)                                                                               \
  {                                                                                                    \
    _Pragma("unroll") for (int s_ = 0; s_ < SUB; ++s_) {                                               \
      bf16x8_t ah[MW], al[MW], b[4];                                                                   \
      _Pragma("unroll") for (int i = 0; i < MW; ++i) {                                                 \
        const int off = tg_sw(wm * 16 * MW + 16 * i + c16, gq);                                        \
        ah[i] = *reinterpret_cast<const bf16x8_t*>(&sAh[buf][s_][off]);                                \
        al[i] = *reinterpret_cast<const bf16x8_t*>(&sAl[buf][s_][off]);                                \
      }                                                                                                \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) b[j] =                                             \
          *reinterpret_cast<const bf16x8_t*>(&sW[buf][s_][tg_sw(wn * 64 + 16 * j + c16, gq)]);         \
      _Pragma("unroll") for (int i = 0; i < MW; ++i) _Pragma("unroll") for (int j = 0; j < 4; ++j) {   \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], b[j], acc[i][j], 0, 0, 0);          \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], b[j], acc[i][j], 0, 0, 0);          \
      }                                                                                                \
    }                                                                                                  \
  }

  f32x4_t acc[MW][4];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int S = gridDim.z, kz = blockIdx.z;
  const int kbeg = kz * (sp.kc / KS), nk = min(K / KS, kbeg + sp.kc / KS);
  QDEC_TG_LOAD(X, kbeg * KS)
  QDEC_TG_STORE(X, 0)
  if constexpr (MW == 4) {
    // 128-row tiles: one step ahead (a second register set would cost the
    // third workgroup per CU)
    __syncthreads();
    for (int kt = kbeg; kt < nk; ++kt) {
      const int buf = (kt - kbeg) & 1;
      if (kt + 1 < nk) QDEC_TG_LOAD(X, (kt + 1) * KS)
      QDEC_TG_MMA(buf)
      if (kt + 1 < nk) QDEC_TG_STORE(X, buf ^ 1)
      __syncthreads();
    }
  } else {
  // step kbeg in LDS buffer 0, step kbeg + 1 in set X (loads past the last
  // step reread it: their stores are skipped)
  QDEC_TG_LOAD(X, min(kbeg + 1, nk - 1) * KS)
  __syncthreads();
  for (int kt = kbeg; kt < nk; kt += 2) {
    // buffer 0 holds step kt, set X step kt + 1
    QDEC_TG_LOAD(Y, min(kt + 2, nk - 1) * KS)
    QDEC_TG_MMA(0)
    if (kt + 1 < nk) QDEC_TG_STORE(X, 1)
    __syncthreads();
    if (kt + 1 >= nk) break;
    // buffer 1 holds step kt + 1, set Y step kt + 2
    QDEC_TG_LOAD(X, min(kt + 3, nk - 1) * KS)
    QDEC_TG_MMA(1)
    if (kt + 2 < nk) QDEC_TG_STORE(Y, 0)
    __syncthreads();
  }
  }
#undef QDEC_TG_LD
#undef QDEC_TG_ST
#undef QDEC_TG_LOAD
#undef QDEC_TG_STORE
#undef QDEC_TG_MMA

  if (S > 1) {
    float* pz = sp.P + (size_t)kz * M * N;
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + 16 * j + c16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * 16 * MW + 16 * i + 4 * gq + e;
          if (row < M) pz[(size_t)row * N + col] = acc[i][j][e];
        }
      }
    return;
  }

#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + c16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 16 * MW + 16 * i + 4 * gq + e;
        const float v = acc[i][j][e];
        if (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SPLIT) {
          const float u = __shfl_xor(v, 8, kWave);
          if (c16 < kGuGroup && row < M) {
            const size_t o = (size_t)row * ldc + (col / 16) * kGuGroup + c16;
            const float z = silu_mul(v, u);
            if (EPI == EPI_SWIGLU) {
              C[o] = z;
            } else {
              // the down projection's operand directly: bf16 hi and lo of the
              // rounded fp32 z (no contraction into the product above)
#pragma clang fp contract(off)
              const uint16_t h = f32_to_bf16_rne(z);
              Zhi[o] = h;
              Zlo[o] = f32_to_bf16_rne(z - bf16_to_f32(h));
            }
          }
        } else if (row < M) {
          const float vb = bias ? v + bias[col] : v;
          if (EPI == EPI_RESID)
            C[(size_t)row * ldc + col] += vb;
          else if (EPI == EPI_RELU)
            C[(size_t)row * ldc + col] = fmaxf(vb, 0.f);
          else
            C[(size_t)row * ldc + col] = vb;
        }
      }
    }
}

// Sum of the S split partials P[z][row][col] in split order, plus bias, into
// C by the epilogue (STORE, RESID or RELU); 4 columns per thread.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int S, int M, int N,
                                                            float* __restrict__ C, int ldc,
                                                            const float* __restrict__ bias) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n4 = (size_t)M * N / 4;
  if (i4 >= n4) return;
  const size_t i = i4 * 4;
  const int row = (int)(i / N), col = (int)(i % N);
  float4 v = *reinterpret_cast<const float4*>(P + i);
  for (int z = 1; z < S; ++z) {
    const float4 t = *reinterpret_cast<const float4*>(P + (size_t)z * M * N + i);
    v.x += t.x;
    v.y += t.y;
    v.z += t.z;
    v.w += t.w;
  }
  if (bias) {
    v.x += bias[col];
    v.y += bias[col + 1];
    v.z += bias[col + 2];
    v.w += bias[col + 3];
  }
  float* c = C + (size_t)row * ldc + col;
  if (EPI == EPI_RESID) {
    c[0] += v.x;
    c[1] += v.y;
    c[2] += v.z;
    c[3] += v.w;
  } else if (EPI == EPI_RELU) {
    c[0] = fmaxf(v.x, 0.f);
    c[1] = fmaxf(v.y, 0.f);
    c[2] = fmaxf(v.z, 0.f);
    c[3] = fmaxf(v.w, 0.f);
  } else {
    c[0] = v.x;
    c[1] = v.y;
    c[2] = v.z;
    c[3] = v.w;
  }
}

// The split sum of splitk_reduce_kernel with the residual epilogue, fused
// with the RMSNorm that follows it: block = one row of N <= 1024 R columns;
// each element x = C + sum of the splits in order is stored to C, then
// x * inv * gain (inv from the row's sum of squares) is written as bf16 hi
// and lo, as rms_split_vec_kernel does.
template <int R>
__global__ __launch_bounds__(256) void splitk_resid_norm_kernel(const float* __restrict__ P, int S, int M, int N,
                                                                float* __restrict__ C, int ldc,
                                                                const float* __restrict__ gain, float eps,
                                                                uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  __shared__ float red[8];
  const int t = blockIdx.x, nc = N / 4;
  float4 v[R];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = threadIdx.x + 256 * r;
    v[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nc) {
      const size_t i = (size_t)t * N + 4 * c;
      float4 a = *reinterpret_cast<const float4*>(P + i);
      for (int z = 1; z < S; ++z) {
        const float4 b = *reinterpret_cast<const float4*>(P + (size_t)z * M * N + i);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
      }
      float* cp = C + (size_t)t * ldc + 4 * c;
      v[r] = make_float4(cp[0] + a.x, cp[1] + a.y, cp[2] + a.z, cp[3] + a.w);
      cp[0] = v[r].x;
      cp[1] = v[r].y;
      cp[2] = v[r].z;
      cp[3] = v[r].w;
    }
    ss = fmaf(v[r].x, v[r].x, fmaf(v[r].y, v[r].y, fmaf(v[r].z, v[r].z, fmaf(v[r].w, v[r].w, ss))));
  }
  const float inv = 1.f / sqrtf(block_sum(ss, red) / (float)N + eps);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = threadIdx.x + 256 * r;
    if (c < nc) {
      const float4 g = reinterpret_cast<const float4*>(gain)[c];
      const float e[4] = {v[r].x * inv * g.x, v[r].y * inv * g.y, v[r].z * inv * g.z, v[r].w * inv * g.w};
      uint16_t h[4], l[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = f32_to_bf16_rne(e[k]);
        l[k] = f32_to_bf16_rne(e[k] - bf16_to_f32(h[k]));
      }
      const size_t o = (size_t)t * N + 4 * c;
      *reinterpret_cast<uint2*>(hi + o) = make_uint2(h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16));
      *reinterpret_cast<uint2*>(lo + o) = make_uint2(l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16));
    }
  }
}

// fp32 weights: C[M, N] (+)= A[M, K] . W[N, K]^T on the vector units.
// Block 16 x 16 threads computes a 32 x 32 tile (2 x 2 per thread); K tiles of
// 16 staged in LDS. For the SwiGLU epilogue the tile's columns hold whole
// interleave groups (32 = 2 groups of 16).
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int M, int K,
                                                        const float* __restrict__ W, int N, float* __restrict__ C,
                                                        int ldc) {
  __shared__ float As[32][17];
  __shared__ float Ws[32][17];
  __shared__ float Cs[32][33];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int idx = threadIdx.x; idx < 32 * 16; idx += 256) {
      const int rr = idx / 16, kk = idx % 16;
      As[rr][kk] = (m0 + rr < M && k0 + kk < K) ? A[(size_t)(m0 + rr) * K + k0 + kk] : 0.f;
      Ws[rr][kk] = (n0 + rr < N && k0 + kk < K) ? W[(size_t)(n0 + rr) * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = fmaf(As[ty * 2 + i][kk], Ws[tx * 2 + j][kk], acc[i][j]);
    __syncthreads();
  }
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) Cs[ty * 2 + i][tx * 2 + j] = acc[i][j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * 16; idx += 256) {
      const int rr = idx / 16, jj = idx % 16;  // 16 outputs per row: 2 groups x 8
      const int grp = jj / kGuGroup, e = jj % kGuGroup;
      const int row = m0 + rr, pc = n0 + grp * 16 + e;
      if (row < M && pc + kGuGroup < N + kGuGroup && pc < N)
        C[(size_t)row * ldc + (pc / 16) * kGuGroup + e] = silu_mul(Cs[rr][grp * 16 + e], Cs[rr][grp * 16 + 8 + e]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = m0 + ty * 2 + i, col = n0 + tx * 2 + j;
        if (row < M && col < N) {
          if (EPI == EPI_RESID)
            C[(size_t)row * ldc + col] += acc[i][j];
          else
            C[(size_t)row * ldc + col] = acc[i][j];
        }
      }
  }
}

template <typename WT>
__global__ void to_f32_kernel(const WT* __restrict__ src, size_t n, float* __restrict__ dst) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = load_w(src, i);
}

// ------------------------------------------------------------------ sampling
// Sampling after the LM head (NCNN "Qwen3ASR ncnn多平台移植", section 1: greedy,
// temperature, top-k, top-p, repetition penalty; section 6: greedy default).
// Order: penalty on the row's history ids, temperature, candidates by (value
// descending, index ascending), top-k, softmax, top-p prefix, inverse CDF at
// the caller's uniform. A candidate travels as one 64-bit key: the
// order-preserving bits of its float32 value above 0xFFFFFFFF - index, so a
// descending sort of keys is exactly that candidate order.

constexpr int kSampleChunk = 1024;  // keys sorted per block

__device__ __forceinline__ unsigned long long cand_key(float v, int idx) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ float cand_value(unsigned long long k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int cand_index(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

// Descending bitonic sort of N keys in LDS by the whole block: each stage
// visits its N / 2 compare-exchange pairs (i, i + j), i with bit j clear, so
// no thread idles.
template <int N>
__device__ void bitonic_desc(unsigned long long* a) {
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < N / 2; t += blockDim.x) {
        const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1));
        const int p = i + j;
        const unsigned long long x = a[i], y = a[p];
        // runs alternate direction so that each k-run ends up descending
        const bool swap = ((i & k) == 0) ? (x < y) : (x > y);
        a[i] = swap ? y : x;
        a[p] = swap ? x : y;
      }
      __syncthreads();
    }
}

// One level of top-k: block (chunk c, row r) sorts kSampleChunk keys and
// writes its first k. Level 0 (RAW) builds the keys from row r's logits: the
// repetition penalty on the row's history ids, then the temperature (inv_t =
// 0 skips it: greedy). Later levels read the previous level's keys.
template <bool RAW>
__global__ __launch_bounds__(512) void topk_level_kernel(const float* __restrict__ logits, int V,
                                                          const unsigned long long* __restrict__ in, int n_in,
                                                          const int32_t* __restrict__ hist, int nh, float rho,
                                                          float temp, int k, unsigned long long* __restrict__ out) {
  __shared__ unsigned long long key[kSampleChunk];
  const int c = blockIdx.x, r = blockIdx.y;
  const int base = c * kSampleChunk;
  const int n = RAW ? V : n_in;
  for (int i = threadIdx.x; i < kSampleChunk; i += blockDim.x) {
    const int e = base + i;
    unsigned long long kk = 0ull;  // below every real key
    if (e < n) {
      if (RAW) {
        float z = logits[(size_t)r * V + e];
        if (temp > 0.f) z = z / temp;
        kk = cand_key(z, e);
      } else {
        kk = in[(size_t)r * n_in + e];
      }
    }
    key[i] = kk;
  }
  if (RAW && nh > 0) {
    __syncthreads();
    // a history id in this chunk: recompute its value from the logit with the
    // penalty (duplicates write the same key)
    for (int t = threadIdx.x; t < nh; t += blockDim.x) {
      const int id = hist[(size_t)r * nh + t];
      if (id >= base && id < base + kSampleChunk && id < V) {
        float z = logits[(size_t)r * V + id];
        z = z > 0.f ? z / rho : z * rho;
        if (temp > 0.f) z = z / temp;
        key[id - base] = cand_key(z, id);
      }
    }
  }
  __syncthreads();
  bitonic_desc<kSampleChunk>(key);
  const int nc = gridDim.x;
  for (int j = threadIdx.x; j < k; j += blockDim.x) out[((size_t)r * nc + c) * k + j] = key[j];
}

// The pick from row r's k candidates (sorted, keys), one wave: float64
// softmax over the candidates, top-p prefix, inverse CDF at u[r].
__global__ __launch_bounds__(64) void sample_pick_kernel(const unsigned long long* __restrict__ cand, int k,
                                                          float top_p, SampleUniforms u, int32_t* __restrict__ tok) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const unsigned long long* c = cand + (size_t)r * k;
  const double z0 = (double)cand_value(c[0]);
  // lane holds candidates 2 lane and 2 lane + 1
  double e[2], cum[2];
  double run = 0.0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * lane + h;
    e[h] = i < k ? exp((double)cand_value(c[i]) - z0) : 0.0;
  }
  // inclusive scan of the lane pairs, then of the lanes
  double s = e[0] + e[1];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(s, o, kWave);
    if (lane >= o) s += t;
  }
  run = s - (e[0] + e[1]);
  cum[0] = run + e[0];
  cum[1] = cum[0] + e[1];
  const double total = __shfl(s, 63, kWave);
  // top-p: n = 1 + the number of leading candidates whose mass stays below top_p
  int n = k;
  if (top_p < 1.f) {
    const double lim = (double)top_p * total;
    const int below = (2 * lane < k && cum[0] < lim ? 1 : 0) + (2 * lane + 1 < k && cum[1] < lim ? 1 : 0);
    int cnt = below;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
    n = min(k, cnt + 1);
  }
  const double mass = __shfl(n - 1 < 2 * lane + 2 ? cum[(n - 1) & 1] : 0.0, (n - 1) / 2, kWave);
  const double target = (double)u.u[r] * mass;
  // first candidate i < n with cum[i] > target
  int first = n - 1;
  int mine = 1 << 30;
  if (2 * lane < n && cum[0] > target) mine = 2 * lane;
  else if (2 * lane + 1 < n && cum[1] > target) mine = 2 * lane + 1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mine = min(mine, __shfl_xor(mine, o, kWave));
  if (mine < n) first = mine;
  if (lane == 0) tok[r] = cand_index(c[first]);
}

}  // namespace

// ================================================================ launchers

hipError_t launch_embed_prefill(const Dims& d, bool bf16, const void* E, const int32_t* ids, int T,
                                const float* audio, int a0, int La, float* X, float* ssq, hipStream_t st) {
  if (bf16)
    embed_prefill_kernel<uint16_t><<<T, 256, 0, st>>>((const uint16_t*)E, d.H, ids, audio, a0, La, X, ssq);
  else
    embed_prefill_kernel<float><<<T, 256, 0, st>>>((const float*)E, d.H, ids, audio, a0, La, X, ssq);
  return hipGetLastError();
}

hipError_t launch_embed_rows(const Dims& d, bool bf16, const void* E, const BatchRows& rows, float* X, float* ssq,
                             hipStream_t st) {
  if (bf16)
    embed_rows_kernel<uint16_t><<<rows.n, 256, 0, st>>>((const uint16_t*)E, d.H, rows, X, ssq);
  else
    embed_rows_kernel<float><<<rows.n, 256, 0, st>>>((const float*)E, d.H, rows, X, ssq);
  return hipGetLastError();
}

hipError_t launch_lm_head(const Dims& d, bool bf16, const void* E, const float* x, const float* gain,
                          float* logits, unsigned long long* key, hipStream_t st) {
  constexpr int ROWS = 8;
  const int blocks = (d.V + 4 * ROWS - 1) / (4 * ROWS);
  const size_t sh = (size_t)(d.H + 64) * sizeof(float);
  if (bf16) {
    const int kch = (d.H / 8 + 63) / 64;
    if (kch == 1)
      lm_head_kernel<uint16_t, ROWS, 1><<<blocks, 256, sh, st>>>((const uint16_t*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else if (kch == 2)
      lm_head_kernel<uint16_t, ROWS, 2><<<blocks, 256, sh, st>>>((const uint16_t*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else if (kch <= 4)
      lm_head_kernel<uint16_t, ROWS, 4><<<blocks, 256, sh, st>>>((const uint16_t*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else if (kch <= 8)
      lm_head_kernel<uint16_t, ROWS, 8><<<blocks, 256, sh, st>>>((const uint16_t*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else
      return hipErrorInvalidValue;
  } else {
    const int kch = (d.H / 4 + 63) / 64;
    if (kch == 1)
      lm_head_kernel<float, ROWS, 1><<<blocks, 256, sh, st>>>((const float*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else if (kch == 2)
      lm_head_kernel<float, ROWS, 2><<<blocks, 256, sh, st>>>((const float*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else if (kch <= 4)
      lm_head_kernel<float, ROWS, 4><<<blocks, 256, sh, st>>>((const float*)E, d.V, d.H, x, gain, d.eps, logits, key);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_argmax_final(const unsigned long long* key, int n, int32_t* out, hipStream_t st) {
  argmax_final_kernel<<<1, 64, 0, st>>>(key, n, out);
  return hipGetLastError();
}

hipError_t launch_argmax_rows(const float* logits, int n, int V, unsigned long long* key, hipStream_t st) {
  const int chunks = std::max(1, std::min(64, (V + 4095) / 4096));
  argmax_rows_kernel<<<dim3(chunks, n), 256, 0, st>>>(logits, V, key);
  return hipGetLastError();
}

hipError_t launch_reset_keys(unsigned long long* key, int n, hipStream_t st) {
  reset_keys_kernel<<<1, 64, 0, st>>>(key, n);
  return hipGetLastError();
}

hipError_t launch_qk_rope_append(const Dims& d, float* qkv, int T, int pos0, const float* q_norm,
                                 const float* k_norm, const float* rope_cos, const float* rope_sin,
                                 const int64_t* page_table, int layer, hipStream_t st) {
  if (d.D == 128 || d.D == 64 || d.D == 32) {
    const int hpb = 4 * (kWave / (d.D / 8));  // heads per 256-thread block
    const dim3 grid((d.NQ + d.NKV + hpb - 1) / hpb, T);
#define QDEC_ROPE_VEC(DD)                                                                                 \
  qk_rope_append_vec_kernel<DD><<<grid, 256, 0, st>>>(qkv, d.qkv(), pos0, d.NQ, d.NKV, d.L, d.eps, q_norm, k_norm, \
                                                      rope_cos, rope_sin, page_table, layer)
    if (d.D == 128)
      QDEC_ROPE_VEC(128);
    else if (d.D == 64)
      QDEC_ROPE_VEC(64);
    else
      QDEC_ROPE_VEC(32);
#undef QDEC_ROPE_VEC
    return hipGetLastError();
  }
  dim3 grid(d.NQ + d.NKV, T);
  qk_rope_append_kernel<<<grid, 64, 0, st>>>(qkv, d.qkv(), pos0, d.NQ, d.NKV, d.D, d.L, d.eps, q_norm, k_norm,
                                             rope_cos, rope_sin, page_table, layer);
  return hipGetLastError();
}

bool attn_small_fits(const Dims& d, int T) {
  const int group = d.NQ / d.NKV;
  return T >= 1 && T <= kSmallT && (d.D == 32 || d.D == 64 || d.D == 128) && (group == 1 || group == 2 || group == 4);
}

hipError_t launch_attn_small(const Dims& d, const float* qkv, int T, const float* q_norm, const float* k_norm,
                             const float* rope_cos, const float* rope_sin, const int64_t* page_table, int layer,
                             float* out, hipStream_t st) {
  if (!attn_small_fits(d, T)) return hipErrorInvalidValue;
  const int group = d.NQ / d.NKV;
  const float qscale = 1.4426950408889634f / sqrtf((float)d.D);  // scores in base 2
  const dim3 grid(d.NKV, (T + kSmallQB - 1) / kSmallQB);
#define QDEC_SMALL_CASE(DD, GG)                                                                             \
  if (d.D == DD && group == GG) {                                                                           \
    attn_small_kernel<DD, GG><<<grid, 512, 0, st>>>(qkv, T, d.NQ, d.NKV, d.L, d.eps, qscale, q_norm, k_norm, \
                                                    rope_cos, rope_sin, page_table, layer, out);            \
    return hipGetLastError();                                                                               \
  }
  QDEC_SMALL_CASE(128, 1)
  QDEC_SMALL_CASE(128, 2)
  QDEC_SMALL_CASE(128, 4)
  QDEC_SMALL_CASE(64, 1)
  QDEC_SMALL_CASE(64, 2)
  QDEC_SMALL_CASE(64, 4)
  QDEC_SMALL_CASE(32, 1)
  QDEC_SMALL_CASE(32, 2)
  QDEC_SMALL_CASE(32, 4)
#undef QDEC_SMALL_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_rows(const Dims& d, const AttnRows& args, int nsplit, hipStream_t st) {
  const int group = d.NQ / d.NKV;
  AttnRows a = args;
  a.L = d.L;
  a.NKV = d.NKV;
  a.ld = d.qkv();
  a.eps = d.eps;
  a.qscale = 1.4426950408889634f / sqrtf((float)d.D);  // scores in base 2
  dim3 grid(d.NKV, nsplit, a.rows.n);
#define QDEC_ATTN_CASE(DD, GG)                                    \
  if (d.D == DD && group == GG) {                                 \
    attn_rows_kernel<DD, GG><<<grid, 256, 0, st>>>(a);            \
  } else
  QDEC_ATTN_CASE(128, 2)
  QDEC_ATTN_CASE(128, 1)
  QDEC_ATTN_CASE(128, 4)
  QDEC_ATTN_CASE(64, 2)
  QDEC_ATTN_CASE(32, 2)
  QDEC_ATTN_CASE(32, 1)
  QDEC_ATTN_CASE(32, 4)
  return hipErrorInvalidValue;
#undef QDEC_ATTN_CASE
  return hipGetLastError();
}

int kv_split_pad(int T) { return (T + 63) / 64 * 64; }

// GQA-2 prompts shorter than this take one query head per attention block
// (512 tokens: 128 blocks in 2 key ranges instead of 64 in 4, whole prefill
// 3.41 -> 3.29 ms; 1024 tokens: 256 blocks and no key-range split instead of
// 128 in 2 ranges, even)
constexpr int kOneQBelow = 2048;

bool attn_prefill_uses_split(const Dims& d) {
  const int group = d.NQ / d.NKV;
  return d.D == fa::D && (group == 1 || group == 2);
}

bool attn_prefill_ropes(const Dims& d) { return attn_prefill_uses_split(d); }

hipError_t launch_attn_prefill(const Dims& d, const float* qkv, int T, float* out, uint16_t* const kv[4],
                               hipStream_t st, uint16_t* out_hi, uint16_t* out_lo, bool causal, SplitK* sk,
                               const QkRope* rope) {
  const int group = d.NQ / d.NKV;
  if ((out_hi != nullptr) != (out_lo != nullptr) || ((out_hi || !causal) && !attn_prefill_uses_split(d)))
    return hipErrorInvalidValue;
  if (rope && rope->norm && !attn_prefill_ropes(d)) return hipErrorInvalidValue;
  const float scale = 1.f / sqrtf((float)d.D);
  if (attn_prefill_uses_split(d)) {
    QkRope rp{};
    if (rope) rp = *rope;
    const int Tp = kv_split_pad(T);
    kv_split_kernel<<<dim3(Tp / kKvTile, d.NKV), 256, 0, st>>>(qkv, T, d.qkv(), d.NQ, d.NKV, kv[0], kv[1], kv[2], kv[3],
                                                          Tp, rp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float qs = scale * 1.4426950408889634f;  // scores in base 2
    // one query head per KV head and a long input: two 16-query blocks per
    // wave, 128 per block (6000 frames of the adaptor: 2.11 -> 1.99 ms; below
    // 1024 positions the halved block count costs more than it saves)
    const bool two = group == 1 && T >= 1024;
    const int qtb = two ? 2 * fa::QT : fa::QT;
    const int nqb = (T + qtb - 1) / qtb, ntile = (T + fa::KT - 1) / fa::KT;
    // fewer than 256 workgroups: split every block's key tiles until about
    // 256 run (at most 8 ranges of at least two tiles), partials merged
    // after; causal blocks also shorten their longest chain of key tiles
    // (the 1024-token prefill: 128 workgroups, 2 ranges, 6.6 -> 5.9 ms)
    // GQA 2 below kOneQBelow positions: one query head per block
    const bool oneq = group == 2 && T < kOneQBelow;
    const int heads = oneq ? d.NQ : d.NKV;  // blocks along y
    int S = 1;
    if (sk && nqb * heads < 256) {
      S = std::min(std::min(8, (256 + nqb * heads - 1) / (nqb * heads)), ntile / 2);
      if (S < 2 || (size_t)S * T * d.NQ * (fa::D + 4) > sk->floats) S = 1;
    }
    float* part = S > 1 ? sk->P : nullptr;
    dim3 grid(nqb, heads, S);
    if (group == 1 && !two)
      attn_prefill_mfma_kernel<1, 1, 0><<<grid, 256, 0, st>>>(qkv, T, d.qkv(), kv[0], kv[1], kv[2], kv[3], Tp, out,
                                                              d.NQ * d.D, qs, out_hi, out_lo, causal ? 1 : 0, part, rp);
    else if (oneq)
      attn_prefill_mfma_kernel<2, 1, 1><<<grid, 256, 0, st>>>(qkv, T, d.qkv(), kv[0], kv[1], kv[2], kv[3], Tp, out,
                                                              d.NQ * d.D, qs, out_hi, out_lo, causal ? 1 : 0, part, rp);
    else if (group == 2)
      attn_prefill_mfma_kernel<2, 1, 0><<<grid, 256, 0, st>>>(qkv, T, d.qkv(), kv[0], kv[1], kv[2], kv[3], Tp, out,
                                                              d.NQ * d.D, qs, out_hi, out_lo, causal ? 1 : 0, part, rp);
    else
      attn_prefill_mfma_kernel<1, 2, 0><<<grid, 256, 0, st>>>(qkv, T, d.qkv(), kv[0], kv[1], kv[2], kv[3], Tp, out,
                                                              d.NQ * d.D, qs, out_hi, out_lo, causal ? 1 : 0, part, rp);
    if (S > 1) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      attn_merge_kernel<<<(T * d.NQ + 7) / 8, 256, 0, st>>>(part, S, T, d.NQ, out, out_hi, out_lo);
    }
    return hipGetLastError();
  }
#define QDEC_PATTN_CASE(DD, GG)                                                                      \
  if (d.D == DD && group == GG) {                                                                    \
    dim3 grid((T + 64 / GG - 1) / (64 / GG), d.NKV);                                                \
    attn_prefill_kernel<DD, GG><<<grid, 256, 0, st>>>(qkv, T, d.qkv(), d.NQ, d.NKV, out, d.NQ * d.D, scale); \
  } else
  QDEC_PATTN_CASE(128, 2)
  QDEC_PATTN_CASE(128, 1)
  QDEC_PATTN_CASE(128, 4)
  QDEC_PATTN_CASE(128, 8)
  QDEC_PATTN_CASE(64, 2)
  QDEC_PATTN_CASE(32, 2)
  QDEC_PATTN_CASE(32, 1)
  QDEC_PATTN_CASE(32, 4)
  return hipErrorInvalidValue;
#undef QDEC_PATTN_CASE
  return hipGetLastError();
}

hipError_t launch_ln_split(const float* X, int T, int K, const float* gain, const float* bias, float eps,
                           uint16_t* hi, uint16_t* lo, hipStream_t st, int ldo) {
  if (ldo == 0) ldo = K;
  if (ldo < K) return hipErrorInvalidValue;
  ln_split_kernel<<<T, 256, 0, st>>>(X, K, gain, bias, eps, hi, lo, ldo);
  return hipGetLastError();
}

hipError_t launch_rms_split(const float* X, int T, int K, const float* gain, float eps, uint16_t* hi,
                            uint16_t* lo, hipStream_t st) {
  if (K % 4 == 0 && K <= 1024)
    rms_split_vec_kernel<1><<<T, 256, 0, st>>>(X, K, gain, eps, hi, lo);
  else if (K % 4 == 0 && K <= 4096)
    rms_split_vec_kernel<4><<<T, 256, 0, st>>>(X, K, gain, eps, hi, lo);
  else
    rms_split_kernel<<<T, 256, 0, st>>>(X, K, gain, eps, hi, lo);
  return hipGetLastError();
}

hipError_t launch_rms_apply(const float* X, int T, int K, const float* gain, float eps, float* out,
                            hipStream_t st) {
  rms_apply_kernel<<<T, 256, 0, st>>>(X, K, gain, eps, out);
  return hipGetLastError();
}


namespace {

struct RowsPlan {
  int nt, tiles, kc, nkc;
};

// 64 output columns per workgroup for the LM head (N >= 65536: 2374 instead
// of 4748 workgroups over the vocabulary; batched decode +1.3%) and for wide
// outputs of at least 33 rows (whose row tiles already give enough
// workgroups: 48-token prefill 1.745 -> 1.72 ms; with 16 rows the same
// width costs 9% of batched decode), 32 for other wide outputs (each A load
// then feeds several column tiles), 16 otherwise; K is split into chunks (multiples of 128,
// one k-step of 32 per wave at least) only until the launch has 128
// workgroups, counting every 16-row tile: the split-K exchange costs more
// than the extra weight parallelism gains beyond that (measured on batched
// decode and 48-token prompts, where 48 rows already give three tiles)
RowsPlan rows_plan(int K, int N, int M) {
  RowsPlan p;
  const int rt = (M + 15) / 16;
  const bool wide = N >= 65536 || (N >= 2048 && rt >= 3);
  p.nt = N % 64 == 0 && wide ? 4 : (N % 32 == 0 && N >= 2048 ? 2 : 1);
  p.tiles = N / (16 * p.nt);
  const int want = std::max(1, (128 + p.tiles * rt - 1) / (p.tiles * rt));
  p.kc = std::max(128, ((K + want - 1) / want + 127) / 128 * 128);
  p.nkc = (K + p.kc - 1) / p.kc;
  return p;
}

template <int MT, int NT, typename WT>
hipError_t rows_dispatch(Epi epi, bool norm, dim3 grid, const RowsGemm& g, hipStream_t st) {
  if (epi == EPI_STORE && norm)
    gemm_rows_kernel<MT, NT, EPI_STORE, true, WT><<<grid, 256, 0, st>>>(g);
  else if (epi == EPI_SWIGLU && norm)
    gemm_rows_kernel<MT, NT, EPI_SWIGLU, true, WT><<<grid, 256, 0, st>>>(g);
  else if (epi == EPI_HEAD && norm)
    gemm_rows_kernel<MT, NT, EPI_HEAD, true, WT><<<grid, 256, 0, st>>>(g);
  else if (epi == EPI_RESID && !norm)
    gemm_rows_kernel<MT, NT, EPI_RESID, false, WT><<<grid, 256, 0, st>>>(g);
  else if (epi == EPI_STORE && !norm)
    gemm_rows_kernel<MT, NT, EPI_STORE, false, WT><<<grid, 256, 0, st>>>(g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool rows_fits(int M, int K, int N) { return M >= 1 && M <= 64 && K >= 32 && K % 32 == 0 && N % 16 == 0; }

int rows_tile_cols(int N) { return rows_plan(32, N, 16).nt * 16; }

size_t rows_partial_floats(int M, int K, int N) {
  const RowsPlan p = rows_plan(K, N, M);
  if (p.nkc == 1) return 0;
  return (size_t)p.nkc * p.tiles * ((M + 15) / 16) * p.nt * 4 * 64;  // 8-byte words
}

int rows_counters(int M, int K, int N) {
  const RowsPlan p = rows_plan(K, N, M);
  return p.nkc == 1 ? 0 : p.tiles * ((M + 15) / 16);
}

hipError_t launch_gemm_rows(Epi epi, bool norm, const RowsGemm& g0, hipStream_t st) {
  if (!rows_fits(g0.M, g0.K, g0.N)) return hipErrorInvalidValue;
  const RowsPlan p = rows_plan(g0.K, g0.N, g0.M);
  if (p.nkc > 1 && (!g0.P || !g0.cnt)) return hipErrorInvalidValue;
  RowsGemm g = g0;
  g.KC = p.kc;
  // one 16-row tile per workgroup: rows past 16 take more workgroups (their
  // weight tiles are read again, mostly from the XCD's L2), not more registers
  const dim3 grid(p.tiles, p.nkc, (g.M + 15) / 16);
  if (g.wf32)
    return p.nt == 4   ? rows_dispatch<1, 4, float>(epi, norm, grid, g, st)
           : p.nt == 2 ? rows_dispatch<1, 2, float>(epi, norm, grid, g, st)
                       : rows_dispatch<1, 1, float>(epi, norm, grid, g, st);
  return p.nt == 4   ? rows_dispatch<1, 4, uint16_t>(epi, norm, grid, g, st)
         : p.nt == 2 ? rows_dispatch<1, 2, uint16_t>(epi, norm, grid, g, st)
                     : rows_dispatch<1, 1, uint16_t>(epi, norm, grid, g, st);
}

namespace {
// Rows per output tile: 128, or 64 when 128-row tiles would give fewer than
// kRows64Below workgroups (about two per CU): with one 4-wave workgroup per
// CU nothing hides the load latency of a K step.
constexpr int kRows64Below = 512;
int tiled_rows(int M, int N) { return (N / tg::BN) * ((M + 127) / 128) < kRows64Below ? 64 : 128; }
int tiled_tiles(int M, int N) {
  const int r = tiled_rows(M, N);
  return (N / tg::BN) * ((M + r - 1) / r);
}
}  // namespace

// The tiled kernel needs M > 64 and whole column tiles, and is taken only with
// at least 128 tiles: below that its few long-running workgroups leave most
// CUs idle and the 64 x 64 small-M kernel is faster (measured on 183- to
// 1024-row inputs: the 512-token prefill 8.05 -> 7.55 ms, the adaptor at 183
// frames 0.49 -> 0.40 ms).
bool gemm_tiled_fits(bool bf16, int M, int K, int N) {
  return bf16 && M > 64 && N % tg::BN == 0 && K % tg::BK == 0 && tiled_tiles(M, N) >= 128;
}

namespace {

// The tiled kernel's plan for a shape: tile rows, splits (1: none) and K per
// split. Below 256 tiles (one workgroup per CU) a workspace lets the K range
// split until about 512 workgroups run (at most 8 splits, at least four K
// steps each), for the epilogues the reduction kernel applies (STORE, RESID,
// RELU); without a split the kernel is taken from 128 tiles on.
struct TiledPlan {
  bool ok;
  int S, kc, rows, sub;
};
// K sub-steps of 32 per barrier: 2 for 64-row tiles when K (and so every
// split's range) is a multiple of 64
int tiled_sub(int rows, int K) { return rows == 64 && K % (2 * tg::BK) == 0 ? 2 : 1; }
TiledPlan tiled_plan(bool bf16, Epi epi, int M, int K, int N, const SplitK* sk) {
  TiledPlan p{false, 1, K, 128, 1};
  if (!bf16 || M <= 64 || N % tg::BN || K % tg::BK) return p;
  p.rows = tiled_rows(M, N);
  p.sub = tiled_sub(p.rows, K);
  const int ks = tg::BK * p.sub;  // K per step
  const int tiles = tiled_tiles(M, N), nk = K / ks;
  p.ok = tiles >= 128;
  if (tiles >= 256 || !sk || (epi != EPI_STORE && epi != EPI_RESID && epi != EPI_RELU)) return p;
  const int S = std::min(std::min(8, (512 + tiles - 1) / tiles), nk * p.sub / 4);
  if (S < 2 || (size_t)S * M * N > sk->floats) return p;
  const int steps = (nk + S - 1) / S;
  p.ok = true;
  p.kc = steps * ks;
  p.S = (nk + steps - 1) / steps;
  return p;
}

}  // namespace

hipError_t launch_gemm_swiglu_split(const uint16_t* A0, const uint16_t* A1, int M, int K, const uint16_t* W, int N,
                                    uint16_t* zhi, uint16_t* zlo, int ldz, hipStream_t st) {
  if (!gemm_tiled_fits(true, M, K, N)) return hipErrorInvalidValue;
  const int rows = tiled_rows(M, N);
  const dim3 grid(N / tg::BN, (M + rows - 1) / rows);
  const TiledSplit t{nullptr, K};
  if (rows == 128)
    gemm_tiled_kernel<EPI_SWIGLU_SPLIT, 4, 1><<<grid, 256, 0, st>>>(A0, A1, M, K, W, N, nullptr, ldz, zhi, zlo, nullptr, t);
  else if (tiled_sub(rows, K) == 2)
    gemm_tiled_kernel<EPI_SWIGLU_SPLIT, 2, 2><<<grid, 256, 0, st>>>(A0, A1, M, K, W, N, nullptr, ldz, zhi, zlo, nullptr, t);
  else
    gemm_tiled_kernel<EPI_SWIGLU_SPLIT, 2, 1><<<grid, 256, 0, st>>>(A0, A1, M, K, W, N, nullptr, ldz, zhi, zlo, nullptr, t);
  return hipGetLastError();
}

hipError_t launch_gemm(bool bf16, Epi epi, const void* A0, const void* A1, int M, int K, const void* W, int N,
                       float* C, int ldc, hipStream_t st, const float* bias, SplitK* sk, RowNorm* norm) {
  if (norm) norm->done = false;
  if ((bias || epi == EPI_RELU) && (!bf16 || epi == EPI_SWIGLU)) return hipErrorInvalidValue;
  const TiledPlan p = tiled_plan(bf16, epi, M, K, N, sk);
  if (p.ok) {
    const dim3 grid(N / tg::BN, (M + p.rows - 1) / p.rows, p.S);
    const uint16_t *hi = (const uint16_t*)A0, *lo = (const uint16_t*)A1, *w = (const uint16_t*)W;
    const TiledSplit t{p.S > 1 ? sk->P : nullptr, p.kc};
#define QDEC_TILED(E, CC, LDC, B)                                                                          \
  do {                                                                                                     \
    if (p.rows == 128)                                                                                     \
      gemm_tiled_kernel<E, 4, 1><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, CC, LDC, nullptr, nullptr, B, t); \
    else if (p.sub == 2)                                                                                   \
      gemm_tiled_kernel<E, 2, 2><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, CC, LDC, nullptr, nullptr, B, t); \
    else                                                                                                   \
      gemm_tiled_kernel<E, 2, 1><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, CC, LDC, nullptr, nullptr, B, t); \
  } while (0)
    if (p.S > 1) {
      // partials first (no epilogue), then the ordered sum with the epilogue
      QDEC_TILED(EPI_STORE, nullptr, N, nullptr);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (epi == EPI_RESID && norm && !bias && N % 4 == 0 && N <= 4096) {
        if (N <= 1024)
          splitk_resid_norm_kernel<1><<<M, 256, 0, st>>>(sk->P, p.S, M, N, C, ldc, norm->gain, norm->eps, norm->hi,
                                                         norm->lo);
        else
          splitk_resid_norm_kernel<4><<<M, 256, 0, st>>>(sk->P, p.S, M, N, C, ldc, norm->gain, norm->eps, norm->hi,
                                                         norm->lo);
        norm->done = true;
        return hipGetLastError();
      }
      const unsigned blocks = (unsigned)(((size_t)M * N / 4 + 255) / 256);
      if (epi == EPI_RESID)
        splitk_reduce_kernel<EPI_RESID><<<blocks, 256, 0, st>>>(sk->P, p.S, M, N, C, ldc, bias);
      else if (epi == EPI_RELU)
        splitk_reduce_kernel<EPI_RELU><<<blocks, 256, 0, st>>>(sk->P, p.S, M, N, C, ldc, bias);
      else
        splitk_reduce_kernel<EPI_STORE><<<blocks, 256, 0, st>>>(sk->P, p.S, M, N, C, ldc, bias);
      return hipGetLastError();
    }
    if (epi == EPI_STORE)
      QDEC_TILED(EPI_STORE, C, ldc, bias);
    else if (epi == EPI_RESID)
      QDEC_TILED(EPI_RESID, C, ldc, bias);
    else if (epi == EPI_RELU)
      QDEC_TILED(EPI_RELU, C, ldc, bias);
    else
      QDEC_TILED(EPI_SWIGLU, C, ldc, nullptr);
#undef QDEC_TILED
    return hipGetLastError();
  }
  if (bf16) {
    if (K % 32 != 0) return hipErrorInvalidValue;
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    const uint16_t *hi = (const uint16_t*)A0, *lo = (const uint16_t*)A1, *w = (const uint16_t*)W;
    if (epi == EPI_STORE)
      gemm_bf16x2_kernel<EPI_STORE><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, C, ldc, bias);
    else if (epi == EPI_RESID)
      gemm_bf16x2_kernel<EPI_RESID><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, C, ldc, bias);
    else if (epi == EPI_RELU)
      gemm_bf16x2_kernel<EPI_RELU><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, C, ldc, bias);
    else
      gemm_bf16x2_kernel<EPI_SWIGLU><<<grid, 256, 0, st>>>(hi, lo, M, K, w, N, C, ldc, nullptr);
  } else {
    dim3 grid((N + 31) / 32, (M + 31) / 32);
    const float *a = (const float*)A0, *w = (const float*)W;
    if (epi == EPI_STORE)
      gemm_f32_kernel<EPI_STORE><<<grid, 256, 0, st>>>(a, M, K, w, N, C, ldc);
    else if (epi == EPI_RESID)
      gemm_f32_kernel<EPI_RESID><<<grid, 256, 0, st>>>(a, M, K, w, N, C, ldc);
    else
      gemm_f32_kernel<EPI_SWIGLU><<<grid, 256, 0, st>>>(a, M, K, w, N, C, ldc);
  }
  return hipGetLastError();
}

hipError_t launch_sample(const float* logits, int n, int V, const int32_t* hist, int nh, float rho, float temp,
                         int top_k, float top_p, const SampleUniforms& u, unsigned long long* buf0,
                         unsigned long long* buf1, int32_t* tok, hipStream_t st) {
  const int k = temp > 0.f ? top_k : 1;
  if (k < 1 || k > kSampleKMax || n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
  int nc = (V + kSampleChunk - 1) / kSampleChunk;
  topk_level_kernel<true><<<dim3(nc, n), 512, 0, st>>>(logits, V, nullptr, 0, hist, nh, rho, temp, k, buf0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long* cur = buf0;
  unsigned long long* nxt = buf1;
  while (nc > 1) {
    const int n_in = nc * k;
    nc = (n_in + kSampleChunk - 1) / kSampleChunk;
    topk_level_kernel<false><<<dim3(nc, n), 512, 0, st>>>(nullptr, 0, cur, n_in, nullptr, 0, 1.f, 0.f, k, nxt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    std::swap(cur, nxt);
  }
  sample_pick_kernel<<<n, 64, 0, st>>>(cur, k, temp > 0.f ? top_p : 1.f, u, tok);
  return hipGetLastError();
}

size_t sample_buffer_words(int V) {
  return (size_t)kMaxBatch * ((V + kSampleChunk - 1) / kSampleChunk) * kSampleKMax;
}

// Fixed scratch of qdec_sample_noalloc: the two candidate-key buffers of
// launch_sample for up to kMaxBatch rows of a vocabulary of at most
// kSampleStaticChunks * kSampleChunk entries (2 x 2.4 MB). Each GPU holds its
// own copy for the life of the process. In host code `scratch` is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress,
// once per device.
constexpr int kSampleStaticChunks = 150;
constexpr size_t kSampleStaticWords = (size_t)kMaxBatch * kSampleStaticChunks * kSampleKMax;
__device__ __align__(256) unsigned long long scratch[2 * kSampleStaticWords];

int sample_static_max_vocab() { return kSampleStaticChunks * kSampleChunk; }

hipError_t sample_static_scratch(unsigned long long** buf0, unsigned long long** buf1) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *buf0 = (unsigned long long*)addr[dev];
  *buf1 = *buf0 + kSampleStaticWords;
  return hipSuccess;
}

hipError_t launch_to_f32(const void* src, bool bf16, size_t n, float* dst, hipStream_t st) {
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  if (bf16)
    to_f32_kernel<uint16_t><<<blocks, 256, 0, st>>>((const uint16_t*)src, n, dst);
  else
    to_f32_kernel<float><<<blocks, 256, 0, st>>>((const float*)src, n, dst);
  return hipGetLastError();
}

// One thread per Q8_0 block: 34 source bytes (fp16 scale, 32 int8 codes) read
// bytewise, since blocks sit at 2-byte alignment only.
__global__ void q8_unpack_kernel(const uint8_t* src, int rows, int K, int kseg, int row0, int gu_half,
                                 int8_t* codes, uint16_t* scales, float* deq) {
  const int nbk = K / kQ8Block, bps = kseg / kQ8Block, nseg = K / kseg, sp = q8_seg_bytes(kseg);
  const size_t total = (size_t)rows * nbk;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / nbk), b = (int)(i % nbk);
    const uint8_t* blk = src + i * kQ8BlockBytes;
    const unsigned short dbits = (unsigned short)(blk[0] | (blk[1] << 8));
    const float d = (float)__builtin_bit_cast(_Float16, dbits);
    const int dr = gu_half < 0 ? row0 + r : (r / kGuGroup) * 2 * kGuGroup + gu_half * kGuGroup + r % kGuGroup;
    int8_t* c = codes + (size_t)dr * K + (size_t)b * kQ8Block;
    float* w = deq + (size_t)dr * K + (size_t)b * kQ8Block;
    for (int j = 0; j < kQ8Block; ++j) {
      const int8_t q = (int8_t)blk[2 + j];
      c[j] = q;
      w[j] = (float)q * d;  // exact: 8 by 11 significant bits
    }
    const size_t so = ((size_t)dr * nseg + b / bps) * sp;
    scales[so / 2 + b % bps] = dbits;
  }
}

hipError_t launch_q8_unpack(const void* src, int rows, int K, int kseg, int row0, int gu_half, int8_t* codes,
                            uint16_t* scales, float* deq, hipStream_t st) {
  if (rows <= 0 || K <= 0 || K % kQ8Block || kseg <= 0 || kseg % kQ8Block || K % kseg) return hipErrorInvalidValue;
  if (gu_half >= 0 && rows % kGuGroup) return hipErrorInvalidValue;
  const size_t total = (size_t)rows * (K / kQ8Block);
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  q8_unpack_kernel<<<blocks, 256, 0, st>>>((const uint8_t*)src, rows, K, kseg, row0, gu_half, codes, scales, deq);
  return hipGetLastError();
}

}  // namespace qdec
