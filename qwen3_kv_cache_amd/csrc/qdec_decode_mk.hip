// Persistent single-launch decode step for gfx950.
//
// One cooperative launch runs a whole decode step of one sequence (NCNN
// "Qwen3ASR ncnn多平台移植", section 5, steps 1-6): embed the token, 28
// Qwen3 blocks (transcribe.cpp "Forward map - funasr_nano", LLM decoder table)
// and the tied LM head with a greedy argmax. One workgroup per CU.
//
// Cross-CU exchange: every phase publishes its output vector as 8-byte words
// (low half = fp32 value, high half = a tag unique to launch, layer and
// phase), written and read with device-scope (sc1) accesses. A consumer polls
// the words it needs until every tag matches, so the exchange is a single
// round trip and no separate barrier exists. Before polling, each CU issues
// the weight loads of the phase it is about to run, so weight latency overlaps
// the wait. Every poll has a time limit: on expiry the launch records an error
// in host-visible memory and all workgroups return.
//
// Phases per layer (row ranges are split evenly over the CUs):
//   A  x -> RMSNorm -> [q|k|v] rows                       (publishes QKV)
//   B  (kv head g, split s): per-head Q/K-RMSNorm + RoPE of the current token,
//      K/V append at pos (split 0), attention over the split's cached positions
//      (+ the current one in the last split)              (publishes partials)
//   B2 only when splits > 2: one CU per query head merges its partials
//   C  O rows + residual                                  (publishes x')
//   D  x' -> RMSNorm -> gate/up rows -> silu(g) * u       (publishes z)
//   E  down rows + residual                               (publishes x'')
// then the final RMSNorm + tied LM head + argmax.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <algorithm>
#include <cmath>

#include "qdec_internal.h"

namespace qdec {
namespace {

constexpr int kWave = 64;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxReg = 8;  // 16-byte weight chunks a lane holds per batch
constexpr unsigned long long kTimeoutTicks = 200000000ull;  // 2 s of the 100 MHz realtime counter
constexpr int kTagsPerLayer = 8;

typedef unsigned long long u64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename WT>
struct Chunk;
template <>
struct Chunk<uint16_t> {
  static constexpr int N = 8;
  u32x4 raw;
  __device__ __forceinline__ void load(const uint16_t* p) { raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
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
  f32x4 raw;
  __device__ __forceinline__ void load(const float* p) { raw = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)); }
  __device__ __forceinline__ float dot(const float* x) const {
    float s = raw.x * x[0];
    s = fmaf(raw.y, x[1], s);
    s = fmaf(raw.z, x[2], s);
    return fmaf(raw.w, x[3], s);
  }
};

template <typename WT>
__device__ __forceinline__ float wload(const WT* p, size_t i);
template <>
__device__ __forceinline__ float wload<uint16_t>(const uint16_t* p, size_t i) { return bf16f(p[i]); }
template <>
__device__ __forceinline__ float wload<float>(const float* p, size_t i) { return p[i]; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ void ll_put(u64* p, float v, unsigned tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ll_get(const u64* p) {
  return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u64 argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((u64)o << 32) | (u64)(0xFFFFFFFFu - (uint32_t)idx);
}

struct MkParams {
  const void* wbuf;      // packed layers (see LayerW); layer l starts at wbuf + l * layer_elems
  size_t layer_elems, off_o, off_gu, off_d;
  const float* nbuf;     // per layer: in_norm[H], post_norm[H], q_norm[D], k_norm[D]
  int norm_elems;
  const void* embed;
  const float* final_norm;
  const float* rope_cos;
  const float* rope_sin;
  int L, H, NQ, NKV, D, F, V;
  float eps, scale;
  const int64_t* page_table;
  int pos, token;
  const int32_t* token_dev;
  int nsplit;
  float* logits;
  int32_t* argmax_out;
  u64* ll;               // exchange words
  size_t o_qkv, o_att, o_atto, o_xb, o_z, o_xa, o_key;
  unsigned tag0;         // tag base of this launch (multiple of 1024)
  int* err;              // host-visible error flag
  int lds_xn, lds_xb, lds_zz, lds_red, lds_att;  // LDS offsets (floats)
};

#ifdef QDEC_MK_TRACE
// timestamp probes of the 100 MHz realtime counter, per CU (diagnostic builds only)
constexpr int kTraceN = 512;
__device__ unsigned long long g_mk_trace[256 * kTraceN];
#define MK_TRACE(idx)                                                                              \
  do {                                                                                             \
    if (tid == 0 && cu < 256) g_mk_trace[cu * kTraceN + (idx)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define MK_TRACE(idx) \
  do {                \
  } while (0)
#endif

struct Ctx {
  u64 t0;
  int* err;
  __device__ bool expired() const { return __builtin_amdgcn_s_memrealtime() - t0 > kTimeoutTicks; }
};

// All threads: wait until src[0..n) carry `tag`, store the values in dst.
// Returns false (block-uniformly) if the time limit expired.
__device__ bool ll_gather(const u64* src, int n, unsigned tag, float* dst, const Ctx& cx, int tid) {
  bool ok = true;
  for (int base = 0; base < n; base += kThreads * 8) {
    unsigned pend = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (base + (int)tid + j * kThreads < n) pend |= 1u << j;
    while (pend && ok) {
      u64 w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (pend & (1u << j)) w[j] = ll_get(src + base + tid + j * kThreads);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((pend & (1u << j)) && (unsigned)(w[j] >> 32) == tag) {
          dst[base + tid + j * kThreads] = __uint_as_float((unsigned)w[j]);
          pend &= ~(1u << j);
        }
      if (pend && cx.expired()) ok = false;
    }
  }
  return __syncthreads_and(ok);
}

__device__ void fail_launch(const Ctx& cx, int tid) {
  if (tid == 0) __hip_atomic_store(cx.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Rows handled by one wave: rows row0 + wave + kWaves * i for i < nrows_w,
// each of K weights; lane owns 16-byte chunks c = lane + 64 j (j < cpl).
template <typename WT>
struct WaveRows {
  static constexpr int VN = Chunk<WT>::N;
  Chunk<WT> reg[kMaxReg];
  int nchunk, cpl, per_batch;  // chunks per row, chunks per lane per row, rows per register batch

  __device__ void setup(int K) {
    nchunk = K / VN;
    cpl = (nchunk + kWave - 1) / kWave;
    per_batch = kMaxReg / cpl;
  }
  // issue loads for rows rows[b*per_batch ..) of this wave (row index via fn)
  template <typename RowFn>
  __device__ void load(const WT* W, int K, int nr, int batch, RowFn rowfn, int lane) {
#pragma unroll
    for (int q = 0; q < kMaxReg; ++q) {
      const int ri = batch * per_batch + q / cpl, j = q % cpl;
      const int c = lane + kWave * j;
      if (q < per_batch * cpl && ri < nr && c < nchunk) reg[q].load(W + (size_t)rowfn(ri) * K + (size_t)c * VN);
    }
  }
  // dot products of the loaded batch with LDS vector x; out[r] for r < per_batch (wave-reduced)
  __device__ void dot(const float* x, int nr, int batch, float* out, int lane) const {
    float accq[kMaxReg];
    int rq[kMaxReg];
#pragma unroll
    for (int q = 0; q < kMaxReg; ++q) {
      rq[q] = q / cpl;
      const int j = q - rq[q] * cpl;
      const int ri = batch * per_batch + rq[q];
      const int c = lane + kWave * j;
      accq[q] = 0.f;
      if (q < per_batch * cpl && ri < nr && c < nchunk) {
        float xv[VN];
#pragma unroll
        for (int i = 0; i < VN; ++i) xv[i] = x[c * VN + i];
        accq[q] = reg[q].dot(xv);
      }
    }
#pragma unroll
    for (int r = 0; r < kMaxReg; ++r) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxReg; ++q) s += (rq[q] == r) ? accq[q] : 0.f;
      out[r] = (r < per_batch) ? wave_sum(s) : 0.f;
    }
  }
};

// Block-wide sum over 512 threads; red has >= kWaves floats.
__device__ float block_sum(float v, float* red, int tid) {
  v = wave_sum(v);
  const int lane = tid % kWave, wave = tid / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += red[i];
  return s;
}

// xn[i] = x[i] * rsqrt(mean(x^2) + eps) * g[i]
__device__ void rms_norm_lds(const float* x, const float* g, int n, float eps, float* xn, float* red, int tid) {
  float ss = 0.f;
  for (int i = tid; i < n; i += kThreads) ss = fmaf(x[i], x[i], ss);
  ss = block_sum(ss, red, tid);
  const float inv = 1.f / sqrtf(ss / (float)n + eps);
  for (int i = tid; i < n; i += kThreads) xn[i] = x[i] * inv * g[i];
  __syncthreads();
}

// Row range of CU `cu` when R rows are split over nb CUs.
__device__ __forceinline__ void cu_rows(int R, int nb, int cu, int& r0, int& r1) {
  const int per = (R + nb - 1) / nb;
  r0 = min(R, cu * per);
  r1 = min(R, r0 + per);
}

template <typename WT, int D, int GROUP>
__global__ __launch_bounds__(kThreads) void decode_mk_kernel(MkParams p) {
  extern __shared__ float sm[];
  const int H = p.H, NQ = p.NQ, NKV = p.NKV, F = p.F;
  const int QKV = (NQ + 2 * NKV) * D;
  float* xa = sm;              // residual stream entering the block [H]
  float* xn = sm + p.lds_xn;   // normalised activations / staged attention partials
  float* xb = sm + p.lds_xb;   // residual after attention [H]
  float* zz = sm + p.lds_zz;   // FFN activations [F], attention output [NQ*D], merge staging
  float* red = sm + p.lds_red; // scratch [128]
  float* att = sm + p.lds_att; // attention scratch
  const int cu = blockIdx.x, nb = gridDim.x;
  Ctx cx{__builtin_amdgcn_s_memrealtime(), p.err};
  u64* LL = p.ll;
  const unsigned tag0 = p.tag0;
  const WT* embed = (const WT*)p.embed;
  const int n_hist = p.pos;  // cached positions 0 .. pos-1
  {
    const int tid = threadIdx.x;
    (void)tid;
    MK_TRACE(0);
  }

  // layer-0 input: the token's embedding row, read by every CU
  {
    int t = p.token_dev ? p.token_dev[0] : p.token;
    t = t < 0 ? 0 : (t >= p.V ? p.V - 1 : t);
    for (int i = threadIdx.x; i < H; i += kThreads) xa[i] = wload(embed, (size_t)t * H + i);
    __syncthreads();
  }

  WaveRows<WT> wr;
  float outv[kMaxReg];
  for (int l = 0; l < p.L; ++l) {
    // thread index made opaque per iteration: keeps index arithmetic from
    // being hoisted out of the layer loop (and held in registers across it)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const WT* Wl = (const WT*)p.wbuf + (size_t)l * p.layer_elems;
    const WT* Wqkv = Wl;
    const WT* Wo = Wl + p.off_o;
    const WT* Wgu = Wl + p.off_gu;
    const WT* Wd = Wl + p.off_d;
    const float* nrm = p.nbuf + (size_t)l * p.norm_elems;
    const float *g_in = nrm, *g_post = nrm + H, *g_q = nrm + 2 * H, *g_k = nrm + 2 * H + D;
    const unsigned tag = tag0 + (unsigned)l * kTagsPerLayer;
    u64* Lqkv = LL + p.o_qkv + (size_t)(l & 1) * QKV;
    u64* Latt = LL + p.o_att + (size_t)(l & 1) * NQ * p.nsplit * (D + 2);
    u64* Latto = LL + p.o_atto + (size_t)(l & 1) * NQ * D;
    u64* Lxb = LL + p.o_xb + (size_t)(l & 1) * H;
    u64* Lz = LL + p.o_z + (size_t)(l & 1) * F;
    u64* Lxa_in = LL + p.o_xa + (size_t)(l & 1) * H;         // written by layer l-1
    u64* Lxa_out = LL + p.o_xa + (size_t)((l + 1) & 1) * H;  // written by this layer

    MK_TRACE(1 + l * 12 + 0);
    // ---------------- A: RMSNorm + QKV rows
    {
      int r0, r1;
      cu_rows(QKV, nb, cu, r0, r1);
      const int nr_cu = r1 - r0;
      const int nr = nr_cu > wave ? (nr_cu - wave + kWaves - 1) / kWaves : 0;
      wr.setup(H);
      auto rowfn = [&](int i) { return r0 + wave + kWaves * i; };
      wr.load(Wqkv, H, nr, 0, rowfn, lane);
      if (l > 0) {
        if (!ll_gather(Lxa_in, H, tag - kTagsPerLayer + 5, xa, cx, tid)) { fail_launch(cx, tid); return; }
      }
      MK_TRACE(1 + l * 12 + 1);
      rms_norm_lds(xa, g_in, H, p.eps, xn, red, tid);
      for (int b = 0; b * wr.per_batch < nr; ++b) {
        if (b > 0) wr.load(Wqkv, H, nr, b, rowfn, lane);
        wr.dot(xn, nr, b, outv, lane);
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < kMaxReg; ++r) {
            const int ri = b * wr.per_batch + r;
            if (r < wr.per_batch && ri < nr) ll_put(Lqkv + rowfn(ri), outv[r], tag + 0);
          }
        }
      }
    }

    MK_TRACE(1 + l * 12 + 2);
    // ---------------- B: attention units (kv head g, split s)
    const int nunits = NKV * p.nsplit;
    if (cu < nunits) {
      const int g = cu / p.nsplit, s = cu % p.nsplit;
      const int sl = (n_hist + p.nsplit - 1) / p.nsplit;
      const int u0 = min(n_hist, s * sl), u1 = min(n_hist, u0 + sl);
      constexpr int DPL = D / 8;
      const int slot = lane / 8, part = lane % 8;
      float* q_l = att;                       // [GROUP][D] normalised, rotated, scaled
      float* k_l = att + GROUP * D;           // [D]
      float* v_l = k_l + D;                   // [D]
      float* wm = v_l + D;                    // [kWaves][GROUP] running max
      float* wl = wm + kWaves * GROUP;        // [kWaves][GROUP] denominators
      float* wo = wl + kWaves * GROUP;        // [kWaves][GROUP][D]
      float* raw = wo + kWaves * GROUP * D;   // [GROUP + 2][D] raw q, k, v of the current token
      // first pass of cached K/V (independent of the current token): issue before polling
      float kv[DPL], vv[DPL];
      auto load_kv = [&](int u) {
        {
          const float* page = reinterpret_cast<const float*>(p.page_table[u / kPage]);
          Dims dd{p.L, 0, 0, NKV, D, 0, 0, 0.f};
          const float* kp = page + page_offset(dd, l, 0, g, u % kPage) + part * DPL;
          const float* vp = page + page_offset(dd, l, 1, g, u % kPage) + part * DPL;
#pragma unroll
          for (int i = 0; i < DPL; i += 4) {
            const float4 a = *reinterpret_cast<const float4*>(kp + i);
            kv[i] = a.x; kv[i + 1] = a.y; kv[i + 2] = a.z; kv[i + 3] = a.w;
            const float4 c = *reinterpret_cast<const float4*>(vp + i);
            vv[i] = c.x; vv[i + 1] = c.y; vv[i + 2] = c.z; vv[i + 3] = c.w;
          }
        }
      };
      if (wave * 8 + slot < u1 - u0) load_kv(u0 + wave * 8 + slot);
      // raw q (GROUP heads), k, v of this kv head
      bool ok = true;
      {
        // q heads g*GROUP .. +GROUP are contiguous; k head g at NQ*D + g*D; v head g at (NQ+NKV)*D + g*D
        for (int i = tid; i < (GROUP + 2) * D; i += kThreads) {
          const int h = i / D, d = i % D;
          const size_t idx = h < GROUP ? (size_t)(g * GROUP + h) * D + d
                                       : (h == GROUP ? (size_t)NQ * D + (size_t)g * D + d
                                                     : (size_t)(NQ + NKV) * D + (size_t)g * D + d);
          u64 w;
          while (true) {
            w = ll_get(Lqkv + idx);
            if ((unsigned)(w >> 32) == tag + 0) break;
            if (cx.expired()) { ok = false; break; }
          }
          if (!ok) break;
          raw[i] = __uint_as_float((unsigned)w);
        }
      }
      if (!__syncthreads_and(ok)) { fail_launch(cx, tid); return; }
      MK_TRACE(1 + l * 12 + 3);
      // per-head RMSNorm + RoPE (waves 0..GROUP: q heads then k); v copied
      if (wave <= GROUP) {
        const float* src = raw + wave * D;
        const float* gg = wave < GROUP ? g_q : g_k;
        const int half = D / 2;
        float a = 0.f, b = 0.f;
        if (lane < half) { a = src[lane]; b = src[lane + half]; }
        const float ss = wave_sum(a * a + b * b);
        const float inv = 1.f / sqrtf(ss / (float)D + p.eps);
        if (lane < half) {
          a = a * inv * gg[lane];
          b = b * inv * gg[lane + half];
          const float c = p.rope_cos[(size_t)p.pos * half + lane], sn = p.rope_sin[(size_t)p.pos * half + lane];
          const float ra = a * c - b * sn, rb = b * c + a * sn;
          if (wave < GROUP) {
            q_l[wave * D + lane] = ra * p.scale;
            q_l[wave * D + lane + half] = rb * p.scale;
          } else {
            k_l[lane] = ra;
            k_l[lane + half] = rb;
          }
        }
      } else if (wave == GROUP + 1) {
        for (int i = lane; i < D; i += kWave) v_l[i] = raw[(GROUP + 1) * D + i];
      }
      __syncthreads();
      if (s == 0) {  // append this position's K and V to the cache
        float* page = reinterpret_cast<float*>(p.page_table[p.pos / kPage]);
        Dims dd{p.L, 0, 0, NKV, D, 0, 0, 0.f};
        for (int i = tid; i < 2 * D; i += kThreads) {
          const int kvsel = i / D, d = i % D;
          page[page_offset(dd, l, kvsel, g, p.pos % kPage) + d] = kvsel ? v_l[d] : k_l[d];
        }
      }
      float qr[GROUP][DPL];
#pragma unroll
      for (int h = 0; h < GROUP; ++h)
#pragma unroll
        for (int i = 0; i < DPL; ++i) qr[h][i] = q_l[h * D + part * DPL + i];
      float m[GROUP], lsum[GROUP], acc[GROUP][DPL];
#pragma unroll
      for (int h = 0; h < GROUP; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[h][i] = 0.f;
      }
      // keys of this split: cached positions [u0, u1), then the current token in the last split
      const int n_cached = u1 - u0;
      const int n_keys = n_cached + (s == p.nsplit - 1 ? 1 : 0);
      for (int kb = wave * 8; kb < n_keys; kb += kWaves * 8) {
        const int ki = kb + slot;
        const bool valid = ki < n_keys;
        if (kb != wave * 8 && ki < n_cached) load_kv(u0 + ki);
        if (!valid) {
#pragma unroll
          for (int i = 0; i < DPL; ++i) kv[i] = vv[i] = 0.f;
        }
        if (valid && ki >= n_cached) {
#pragma unroll
          for (int i = 0; i < DPL; ++i) {
            kv[i] = k_l[part * DPL + i];
            vv[i] = v_l[part * DPL + i];
          }
        }
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
          float sc = 0.f;
#pragma unroll
          for (int i = 0; i < DPL; ++i) sc = fmaf(qr[h][i], kv[i], sc);
          sc += __shfl_xor(sc, 1, kWave);
          sc += __shfl_xor(sc, 2, kWave);
          sc += __shfl_xor(sc, 4, kWave);
          if (!valid) sc = -INFINITY;
          float mx = fmaxf(sc, __shfl_xor(sc, 8, kWave));
          mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
          mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
          const float mn = fmaxf(m[h], mx);
          const float alpha = expf(m[h] - mn);
          const float pr = valid ? expf(sc - mn) : 0.f;
          float ps = pr + __shfl_xor(pr, 8, kWave);
          ps += __shfl_xor(ps, 16, kWave);
          ps += __shfl_xor(ps, 32, kWave);
          lsum[h] = lsum[h] * alpha + ps;
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc[h][i] = fmaf(pr, vv[i], acc[h][i] * alpha);
          m[h] = mn;
        }
      }
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
          for (int i = 0; i < DPL; ++i) wo[(wave * GROUP + h) * D + part * DPL + i] = acc[h][i];
      }
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
          wm[wave * GROUP + h] = m[h];
          wl[wave * GROUP + h] = lsum[h];
        }
      }
      __syncthreads();
      for (int idx = tid; idx < GROUP * (D + 2); idx += kThreads) {
        const int h = idx / (D + 2), e = idx % (D + 2);
        float M = -INFINITY;
        for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, wm[w2 * GROUP + h]);
        float val = 0.f;
        if (e == 0) {
          val = M;
        } else {
          for (int w2 = 0; w2 < kWaves; ++w2) {
            const float mw = wm[w2 * GROUP + h];
            const float f = (mw == -INFINITY) ? 0.f : expf(mw - M);
            val = fmaf(f, e == 1 ? wl[w2 * GROUP + h] : wo[(w2 * GROUP + h) * D + (e - 2)], val);
          }
        }
        ll_put(Latt + ((size_t)(g * GROUP + h) * p.nsplit + s) * (D + 2) + e, val, tag + 1);
      }
    }

    // ---------------- B2: merge splits per query head (long contexts)
    const bool merged = p.nsplit > 2;
    if (merged && cu < NQ) {
      const int h = cu;
      const int nw = p.nsplit * (D + 2);
      if (!ll_gather(Latt + (size_t)h * nw, nw, tag + 1, zz, cx, tid)) { fail_launch(cx, tid); return; }
      for (int d = tid; d < D; d += kThreads) {
        float M = -INFINITY;
        for (int s2 = 0; s2 < p.nsplit; ++s2) M = fmaxf(M, zz[s2 * (D + 2)]);
        float o = 0.f, lt = 0.f;
        for (int s2 = 0; s2 < p.nsplit; ++s2) {
          const float ms = zz[s2 * (D + 2)];
          const float f = (ms == -INFINITY) ? 0.f : expf(ms - M);
          o = fmaf(f, zz[s2 * (D + 2) + 2 + d], o);
          lt = fmaf(f, zz[s2 * (D + 2) + 1], lt);
        }
        ll_put(Latto + (size_t)h * D + d, o / lt, tag + 2);
      }
      __syncthreads();
    }

    MK_TRACE(1 + l * 12 + 4);
    // ---------------- C: O rows + residual
    {
      int r0, r1;
      cu_rows(H, nb, cu, r0, r1);
      const int nr_cu = r1 - r0;
      const int nr = nr_cu > wave ? (nr_cu - wave + kWaves - 1) / kWaves : 0;
      const int K = NQ * D;
      wr.setup(K);
      auto rowfn = [&](int i) { return r0 + wave + kWaves * i; };
      wr.load(Wo, K, nr, 0, rowfn, lane);
      // attention output [NQ*D] into zz
      if (merged) {
        if (!ll_gather(Latto, K, tag + 2, zz, cx, tid)) { fail_launch(cx, tid); return; }
      } else {
        const int nw = NQ * p.nsplit * (D + 2);
        float* parts = xn;  // reuse: needs NQ * nsplit * (D + 2) <= staging size (checked on the host)
        if (!ll_gather(Latt, nw, tag + 1, parts, cx, tid)) { fail_launch(cx, tid); return; }
        for (int idx = tid; idx < K; idx += kThreads) {
          const int h = idx / D, d = idx % D;
          const float* ph = parts + (size_t)h * p.nsplit * (D + 2);
          float M = -INFINITY;
          for (int s2 = 0; s2 < p.nsplit; ++s2) M = fmaxf(M, ph[s2 * (D + 2)]);
          float o = 0.f, lt = 0.f;
          for (int s2 = 0; s2 < p.nsplit; ++s2) {
            const float ms = ph[s2 * (D + 2)];
            const float f = (ms == -INFINITY) ? 0.f : expf(ms - M);
            o = fmaf(f, ph[s2 * (D + 2) + 2 + d], o);
            lt = fmaf(f, ph[s2 * (D + 2) + 1], lt);
          }
          zz[idx] = o / lt;
        }
        __syncthreads();
      }
      MK_TRACE(1 + l * 12 + 5);
      for (int b = 0; b * wr.per_batch < nr; ++b) {
        if (b > 0) wr.load(Wo, K, nr, b, rowfn, lane);
        wr.dot(zz, nr, b, outv, lane);
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < kMaxReg; ++r) {
            const int ri = b * wr.per_batch + r;
            if (r < wr.per_batch && ri < nr) {
              const int row = rowfn(ri);
              ll_put(Lxb + row, xa[row] + outv[r], tag + 3);
            }
          }
        }
      }
    }

    MK_TRACE(1 + l * 12 + 6);
    // ---------------- D: RMSNorm + gate/up rows + SiLU * up
    {
      int z0, z1;
      cu_rows(F, nb, cu, z0, z1);
      const int nz = z1 - z0;           // z outputs of this CU
      const int nrow = 2 * nz;          // gate and up rows, interleaved: item i -> z0 + i/2, gate if even
      const int nr = nrow > wave ? (nrow - wave + kWaves - 1) / kWaves : 0;
      wr.setup(H);
      auto rowfn = [&](int i) {
        const int it = wave + kWaves * i;
        const int j = z0 + it / 2;
        return (j / kGuGroup) * 2 * kGuGroup + ((it & 1) ? kGuGroup : 0) + j % kGuGroup;
      };
      wr.load(Wgu, H, nr, 0, rowfn, lane);
      if (!ll_gather(Lxb, H, tag + 3, xb, cx, tid)) { fail_launch(cx, tid); return; }
      MK_TRACE(1 + l * 12 + 7);
      rms_norm_lds(xb, g_post, H, p.eps, xn, red, tid);
      float* rowsum = red + 2 * kWaves;  // [2 * nz] <= 96 floats
      for (int b = 0; b * wr.per_batch < nr; ++b) {
        if (b > 0) wr.load(Wgu, H, nr, b, rowfn, lane);
        wr.dot(xn, nr, b, outv, lane);
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < kMaxReg; ++r) {
            const int ri = b * wr.per_batch + r;
            if (r < wr.per_batch && ri < nr) rowsum[wave + kWaves * ri] = outv[r];
          }
        }
      }
      __syncthreads();
      if ((int)tid < nz) {
        const float gt = rowsum[2 * tid], up = rowsum[2 * tid + 1];
        ll_put(Lz + z0 + tid, gt / (1.f + expf(-gt)) * up, tag + 4);
      }
    }

    MK_TRACE(1 + l * 12 + 8);
    // ---------------- E: down rows + residual
    {
      int r0, r1;
      cu_rows(H, nb, cu, r0, r1);
      const int nr_cu = r1 - r0;
      const int nr = nr_cu > wave ? (nr_cu - wave + kWaves - 1) / kWaves : 0;
      wr.setup(F);
      auto rowfn = [&](int i) { return r0 + wave + kWaves * i; };
      wr.load(Wd, F, nr, 0, rowfn, lane);
      if (!ll_gather(Lz, F, tag + 4, zz, cx, tid)) { fail_launch(cx, tid); return; }
      MK_TRACE(1 + l * 12 + 9);
      for (int b = 0; b * wr.per_batch < nr; ++b) {
        if (b > 0) wr.load(Wd, F, nr, b, rowfn, lane);
        wr.dot(zz, nr, b, outv, lane);
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < kMaxReg; ++r) {
            const int ri = b * wr.per_batch + r;
            if (r < wr.per_batch && ri < nr) {
              const int row = rowfn(ri);
              ll_put(Lxa_out + row, xb[row] + outv[r], tag + 5);
            }
          }
        }
      }
    }
  }

  // ---------------- final RMSNorm + tied LM head + argmax
  {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const unsigned tag_last = tag0 + (unsigned)(p.L - 1) * kTagsPerLayer + 5;
    int r0, r1;
    cu_rows(p.V, nb, cu, r0, r1);
    const int nr_cu = r1 - r0;
    const int nr = nr_cu > wave ? (nr_cu - wave + kWaves - 1) / kWaves : 0;
    WaveRows<WT> wr2;
    wr.setup(H);
    wr2.setup(H);
    auto rowfn = [&](int i) { return r0 + wave + kWaves * i; };
    wr.load(embed, H, nr, 0, rowfn, lane);
    if (!ll_gather(LL + p.o_xa + (size_t)(p.L & 1) * H, H, tag_last, xa, cx, tid)) { fail_launch(cx, tid); return; }
    MK_TRACE(400);
    rms_norm_lds(xa, p.final_norm, H, p.eps, xn, red, tid);
    u64 best = 0ull;
    const int nbatch = (nr + wr.per_batch - 1) / wr.per_batch;
    for (int b = 0; b < nbatch; b += 2) {
      if (b + 1 < nbatch) wr2.load(embed, H, nr, b + 1, rowfn, lane);
      for (int half = 0; half < 2 && b + half < nbatch; ++half) {
        const int bb = b + half;
        if (half == 0) wr.dot(xn, nr, bb, outv, lane);
        else wr2.dot(xn, nr, bb, outv, lane);
        if (half == 0 && b + 2 < nbatch) wr.load(embed, H, nr, b + 2, rowfn, lane);
#pragma unroll
        for (int r = 0; r < kMaxReg; ++r) {
          const int ri = bb * wr.per_batch + r;
          if (r < wr.per_batch && ri < nr) {
            const int row = rowfn(ri);
            if (p.logits && lane == 0) p.logits[row] = outv[r];
            const u64 k = argmax_key(outv[r], row);
            best = k > best ? k : best;
          }
        }
      }
    }
    MK_TRACE(401);
    // block max -> this CU's words in the key table (hi and lo halves tagged)
    u64* bk = reinterpret_cast<u64*>(red);
    __syncthreads();
    if (lane == 0) bk[wave] = best;
    __syncthreads();
    u64* Lkey = LL + p.o_key;
    const unsigned ktag = tag0 + 1023u;
    if (tid == 0) {
      u64 b2 = bk[0];
      for (int i = 1; i < kWaves; ++i) b2 = bk[i] > b2 ? bk[i] : b2;
      ll_put(Lkey + 2 * cu, __uint_as_float((unsigned)(b2 >> 32)), ktag);
      ll_put(Lkey + 2 * cu + 1, __uint_as_float((unsigned)b2), ktag);
    }
    // CU 0 reduces the table and writes the token
    if (cu == 0) {
      float* kw = zz;  // 2 * nb floats (bit patterns)
      if (!ll_gather(Lkey, 2 * nb, ktag, kw, cx, tid)) { fail_launch(cx, tid); return; }
      MK_TRACE(402);
      if (tid == 0) {
        u64 b3 = 0ull;
        for (int i = 0; i < nb; ++i) {
          const u64 k = ((u64)__float_as_uint(kw[2 * i]) << 32) | (u64)__float_as_uint(kw[2 * i + 1]);
          b3 = k > b3 ? k : b3;
        }
        p.argmax_out[0] = (int32_t)(0xFFFFFFFFu - (uint32_t)(b3 & 0xFFFFFFFFull));
      }
    }
  }
}

}  // namespace

#ifdef QDEC_MK_TRACE
extern "C" int qdec_debug_trace(unsigned long long* host, int n) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_mk_trace), sizeof(unsigned long long) * (size_t)n, 0,
                                  hipMemcpyDeviceToHost);
}
#endif

// ---------------------------------------------------------------- launcher

// LDS layout (floats): xa[H] | xn[stage] | xb[H] | zz[zsize] | red[128] | att[...]
struct MkLayout {
  int xn, xb, zz, red, att, total;
};
MkLayout mk_layout(const Dims& d, int nsplit) {
  const int group = d.NQ / d.NKV;
  const bool merged = nsplit > 2;
  const int stage = std::max(std::max(d.H, d.NQ * d.D), merged ? 0 : d.NQ * nsplit * (d.D + 2));
  const int zsize = std::max(std::max(d.F, d.NQ * d.D), std::max(nsplit * (d.D + 2), 2 * 1024));
  const int attn = group * d.D + 2 * d.D + 2 * kWaves * group + kWaves * group * d.D + (group + 2) * d.D;
  MkLayout o;
  o.xn = d.H;
  o.xb = o.xn + stage;
  o.zz = o.xb + d.H;
  o.red = o.zz + zsize;
  o.att = o.red + 128;
  o.total = o.att + attn;
  return o;
}

size_t mk_lds_bytes(const Dims& d, int nsplit) { return (size_t)mk_layout(d, nsplit).total * sizeof(float); }

hipError_t launch_decode_mk(const MkLaunch& a, hipStream_t st) {
  MkParams p{};
  p.wbuf = a.wbuf;
  p.layer_elems = a.layer_elems;
  p.off_o = a.off_o;
  p.off_gu = a.off_gu;
  p.off_d = a.off_d;
  p.nbuf = a.nbuf;
  p.norm_elems = a.norm_elems;
  p.embed = a.embed;
  p.final_norm = a.final_norm;
  p.rope_cos = a.rope_cos;
  p.rope_sin = a.rope_sin;
  const Dims& d = a.d;
  p.L = d.L; p.H = d.H; p.NQ = d.NQ; p.NKV = d.NKV; p.D = d.D; p.F = d.F; p.V = d.V;
  p.eps = d.eps;
  p.scale = 1.f / sqrtf((float)d.D);
  p.page_table = a.page_table;
  p.pos = a.pos;
  p.token = a.token;
  p.token_dev = a.token_dev;
  p.nsplit = a.nsplit;
  p.logits = a.logits;
  p.argmax_out = a.argmax_out;
  p.ll = a.ll;
  p.o_qkv = a.o_qkv; p.o_att = a.o_att; p.o_atto = a.o_atto; p.o_xb = a.o_xb; p.o_z = a.o_z; p.o_xa = a.o_xa;
  p.o_key = a.o_key;
  p.tag0 = a.tag0;
  p.err = a.err;
  const MkLayout lay = mk_layout(d, a.nsplit);
  p.lds_xn = lay.xn; p.lds_xb = lay.xb; p.lds_zz = lay.zz; p.lds_red = lay.red; p.lds_att = lay.att;
  const size_t sh = (size_t)lay.total * sizeof(float);
  void* args[] = {&p};
  const int group = d.NQ / d.NKV;
  const void* fn = nullptr;
#define QDEC_MK_CASE(WT, DD, GG) \
  if (d.D == DD && group == GG) fn = (const void*)decode_mk_kernel<WT, DD, GG>;
  if (a.bf16) {
    QDEC_MK_CASE(uint16_t, 128, 2)
    QDEC_MK_CASE(uint16_t, 128, 1)
    QDEC_MK_CASE(uint16_t, 128, 4)
    QDEC_MK_CASE(uint16_t, 128, 8)
    QDEC_MK_CASE(uint16_t, 64, 2)
    QDEC_MK_CASE(uint16_t, 32, 2)
    QDEC_MK_CASE(uint16_t, 32, 4)
  } else {
    QDEC_MK_CASE(float, 128, 2)
    QDEC_MK_CASE(float, 64, 2)
    QDEC_MK_CASE(float, 32, 2)
    QDEC_MK_CASE(float, 32, 4)
    QDEC_MK_CASE(float, 32, 1)
  }
#undef QDEC_MK_CASE
  if (!fn) return hipErrorInvalidValue;
  return hipLaunchCooperativeKernel(fn, dim3(a.nblocks), dim3(kThreads), args, (unsigned)sh, st);
}

hipError_t mk_prepare(bool bf16, const Dims& d, size_t lds_max, int* max_blocks_per_cu) {
  const int group = d.NQ / d.NKV;
  const void* fn = nullptr;
#define QDEC_MK_CASE(WT, DD, GG) \
  if (d.D == DD && group == GG) fn = (const void*)decode_mk_kernel<WT, DD, GG>;
  if (bf16) {
    QDEC_MK_CASE(uint16_t, 128, 2)
    QDEC_MK_CASE(uint16_t, 128, 1)
    QDEC_MK_CASE(uint16_t, 128, 4)
    QDEC_MK_CASE(uint16_t, 128, 8)
    QDEC_MK_CASE(uint16_t, 64, 2)
    QDEC_MK_CASE(uint16_t, 32, 2)
    QDEC_MK_CASE(uint16_t, 32, 4)
  } else {
    QDEC_MK_CASE(float, 128, 2)
    QDEC_MK_CASE(float, 64, 2)
    QDEC_MK_CASE(float, 32, 2)
    QDEC_MK_CASE(float, 32, 4)
    QDEC_MK_CASE(float, 32, 1)
  }
#undef QDEC_MK_CASE
  if (!fn) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(max_blocks_per_cu, fn, kThreads, lds_max);
}

}  // namespace qdec
