// Persistent decode for gfx950: one cooperative launch runs one or more
// greedy decode steps of one sequence (NCNN "Qwen3ASR ncnn多平台移植", section
// 5, steps 1-6): embed the token, the Qwen3 blocks (transcribe.cpp "Forward map
// - funasr_nano", LLM decoder table) and the tied LM head with a greedy argmax
// whose token feeds the next step.
//
// Placement. One workgroup per CU. A launch of nb workgroups places workgroup b
// on XCD b % 8, so workgroups are grouped as (x = b % 8, rank r = b / 8), R =
// nb / 8 ranks per group. KV head g is owned by group g: its Q/K/V rows, its
// attention and its slice of the O projection stay inside one XCD. The FFN is
// split by z slices, one per group, and the down projection is split along the
// same slices. A layer then needs two exchanges that span the whole chip (O
// partials and down partials, both summed by every CU in a fixed order so all
// copies of the residual stream are bit-identical) and two or three inside a
// group. Correctness never depends on the placement, only speed: every
// cross-CU word uses device scope.
//
// Exchange. A phase publishes each output as an 8-byte word: fp32 value in the
// low half, a tag unique to (launch, step, layer, phase) in the high half,
// stored and loaded as device-scope relaxed atomics. A consumer polls until
// every word it needs carries the expected tag. Regions are double-buffered by
// layer parity. Every wait has a time limit; on expiry the launch raises a
// host-visible error flag and all workgroups return.
//
// Two roles per workgroup. A wave's vector-memory counter retires loads in
// issue order, so a load needed now cannot complete before an earlier
// prefetch. Waves 0-3 (memory waves) therefore hold the weights: they issue
// each phase's weight loads one or two phases ahead and compute the dot
// products. Waves 4-7 (exchange waves) issue only latency-critical loads: the
// exchange polls, norm gains, RoPE rows and the KV cache; they also run the
// norms, Q/K-norm + RoPE and attention. The roles meet at workgroup barriers.
//
// Phases of layer l for workgroup (x, r); G = n_q / n_kv query heads per KV
// head, QD = G * D, FS = ffn / 8:
//   A (x < n_kv) x <- x + sum of the previous layer's down partials;
//                RMSNorm; rows [a0, a1) of KV head x's (G + 2) * D Q/K/V rows
//   B (x < n_kv) Q/K-RMSNorm + RoPE of the current token; K/V append (rank 0);
//                attention of the G query heads, either whole in every rank
//                (short history) or split over ranks with partials (m, l, o)
//   C (x < n_kv) rows [c0, c1) of Wo[:, x*QD : (x+1)*QD] . o_x  (O partial of group x)
//   D (all)      x' = x + sum of O partials; RMSNorm; gate/up rows of z
//                indices x*FS + [z0, z1); z = silu(gate) * up
//   E (all)      rows [e0, e1) of Wd[:, x*FS : (x+1)*FS] . z_x (down partial of group x)
// After the last layer: final RMSNorm, the tied LM head over rows split across
// all workgroups, and a greedy argmax (lowest index among equal maxima).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "qdec_internal.h"

namespace qdec {
namespace {

typedef unsigned long long u64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kMemWaves = 4;              // waves 0-3: weights and dot products
constexpr int kExWaves = kWaves - kMemWaves;
constexpr int kEx = kExWaves * kWave;     // exchange threads
constexpr int kExBase = kMemWaves * kWave;  // first exchange thread
constexpr int kGroups = 8;                // XCDs
constexpr u64 kWaitTicks = 200000000ull;  // 2 s of the 100 MHz realtime counter
constexpr int kTagSlots = 8;              // tags per (step, layer)
enum { PH_Q = 0, PH_ATT = 1, PH_O = 2, PH_Z = 3, PH_X = 4, PH_KEY = 5 };

__device__ __forceinline__ u64 now() { return __builtin_amdgcn_s_memrealtime(); }

#ifdef QDEC_TRACE
// Diagnostic builds only: realtime-counter stamps at phase boundaries of the
// first step of a launch, per workgroup (taken by the first exchange thread).
constexpr int kTraceN = 512;
__device__ u64 g_trace[2048 * kTraceN];
#define TRACE(step, idx)                                                                                 \
  do {                                                                                                   \
    if ((step) == 0 && tid == kExBase && (idx) < kTraceN) g_trace[blockIdx.x * kTraceN + (idx)] = now(); \
  } while (0)
// the same from the first memory-wave thread
#define TRACEM(step, idx)                                                                       \
  do {                                                                                          \
    if ((step) == 0 && tid0 == 0 && (idx) >= 0 && (idx) < kTraceN) g_trace[blockIdx.x * kTraceN + (idx)] = now(); \
  } while (0)
#else
#define TRACE(step, idx) \
  do {                   \
  } while (0)
#define TRACEM(step, idx) \
  do {                    \
  } while (0)
#endif

__device__ __forceinline__ void put(u64* p, float v, unsigned tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 get(const u64* p) {
  return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(u64 w, unsigned tag) { return (unsigned)(w >> 32) == tag; }
__device__ __forceinline__ float val(u64 w) { return __uint_as_float((unsigned)w); }

// Cross-lane steps on the VALU (DPP and the gfx950 permlane swaps) instead of
// LDS-routed shuffles. dpp(v, ctrl) returns the value of the lane selected by
// the DPP control within each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each 16
constexpr int kDppXor8 = 0x128;       // row_ror:8, i.e. lane i <-> i ^ 8 within each 16
// (value of lane i, value of lane i ^ 16) and (lane i, lane i ^ 32) as an
// ordered pair (lower lane first), so sums and maxima are bit-identical in both lanes
__device__ __forceinline__ float sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over the 64 lanes; every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return sum32(sum16(v));
}

__device__ __forceinline__ u64 argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((u64)o << 32) | (u64)(0xFFFFFFFFu - (uint32_t)idx);
}

// even split of n items over `parts`: [s, e) of part i
__device__ __forceinline__ void split(int n, int parts, int i, int& s, int& e) {
  const int per = (n + parts - 1) / parts;
  s = min(n, i * per);
  e = min(n, s + per);
}

struct DecParams {
  const void* wbuf;  // packed layers: layer l at wbuf + l * layer_elems (see LayerW)
  size_t layer_elems, off_o, off_gu, off_d;
  const float* nbuf;  // per layer: in_norm[H], post_norm[H], q_norm[D], k_norm[D]
  int norm_elems;
  const void* embed;
  const float* final_norm;
  const float* rope_cos;
  const float* rope_sin;
  const int64_t* page_table;
  int L, H, NQ, NKV, F, V;
  float eps, scale;
  int pos0, nsteps, token;
  const int32_t* token_dev;
  float* logits;        // [nsteps, V] or null
  int32_t* tokens_out;  // [nsteps]
  u64* ll;
  size_t o_q, o_att, o_o, o_z, o_x, o_key;
  unsigned tag0;
  int* err;
  int R;              // ranks per group
  int nsplit_max;     // attention splits per group
  int whole_max;      // cached positions up to which each rank runs the whole attention
  int lds_x, lds_xn, lds_stage, lds_att, lds_red, lds_rbuf, lds_lgb, lds_ring;
};

// ------------------------------------------------------------------ waits
// All waits are called by every thread of the workgroup (they end in a
// barrier); only threads with `act` (the exchange waves) poll. et = exchange
// thread index in [0, kEx).

// x[e] += sum_{q < P} W[q * n + e] for e < n (P <= 8), in that order.
template <int NE>
__device__ __forceinline__ bool gather_sum(bool act, const u64* W, int P, int n, unsigned tag, float* x, int et) {
  bool ok = true;
  if (act) {
    const u64 t0 = now();
    u64 w[NE][kGroups];
    while (true) {
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int e = min(et + k * kEx, n - 1);
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
          if (q < P) w[k][q] = get(W + (size_t)q * n + e);
      }
      bool done = true;
#pragma unroll
      for (int k = 0; k < NE; ++k)
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
          if (q < P) done = done && tagged(w[k][q], tag);
      if (done) break;
      if (now() - t0 > kWaitTicks) {
        ok = false;
        break;
      }
    }
    if (ok) {
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int e = et + k * kEx;
        if (e < n) {
          float s = x[e];
#pragma unroll
          for (int q = 0; q < kGroups; ++q)
            if (q < P) s += val(w[k][q]);
          x[e] = s;
        }
      }
    }
  }
  return __syncthreads_and(ok);
}

// dst[i] = value of W[i] for i < n (n <= J * kEx).
template <int J>
__device__ __forceinline__ bool gather_vec(bool act, const u64* W, int n, unsigned tag, float* dst, int et) {
  bool ok = true;
  if (act) {
    const u64 t0 = now();
    u64 w[J];
    while (true) {
#pragma unroll
      for (int j = 0; j < J; ++j) w[j] = get(W + min(et + j * kEx, n - 1));
      bool done = true;
#pragma unroll
      for (int j = 0; j < J; ++j) done = done && tagged(w[j], tag);
      if (done) break;
      if (now() - t0 > kWaitTicks) {
        ok = false;
        break;
      }
    }
    if (ok) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (et + j * kEx < n) dst[et + j * kEx] = val(w[j]);
    }
  }
  return __syncthreads_and(ok);
}

__device__ __forceinline__ bool gather_any(bool act, const u64* W, int n, unsigned tag, float* dst, int et) {
  if (n <= 2 * kEx) return gather_vec<2>(act, W, n, tag, dst, et);
  if (n <= 8 * kEx) return gather_vec<8>(act, W, n, tag, dst, et);
  return gather_vec<32>(act, W, n, tag, dst, et);
}

__device__ __forceinline__ void fail_launch(int* err, int tid) {
  if (tid == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float block_sum(float v, float* red, int tid) {
  v = wave_sum(v);
  __syncthreads();
  if (tid % kWave == 0) red[tid / kWave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += red[i];
  return s;
}

// xn[i] = x[i] / sqrt(mean(x^2) + eps) * g[i]; elementwise work by the `act` threads.
__device__ __forceinline__ void rms_norm(bool act, const float* x, const float* g, int n, float eps, float* xn,
                                         float* red, int tid, int et) {
  float ss = 0.f;
  if (act)
    for (int i = et; i < n; i += kEx) ss = fmaf(x[i], x[i], ss);
  ss = block_sum(ss, red, tid);
  const float inv = 1.f / sqrtf(ss / (float)n + eps);
  if (act)
    for (int i = et; i < n; i += kEx) xn[i] = x[i] * inv * g[i];
  __syncthreads();
}

template <typename WT>
__device__ __forceinline__ float wload(const WT* p, size_t i);
template <>
__device__ __forceinline__ float wload<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
template <>
__device__ __forceinline__ float wload<float>(const float* p, size_t i) { return p[i]; }

// --------------------------------------------------------------- weights

template <typename WT>
__device__ __forceinline__ float dot_chunk(const u32x4& raw, const float* x);
template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(const u32x4& raw, const float* x) {
  const float4 a = *reinterpret_cast<const float4*>(x);
  const float4 b = *reinterpret_cast<const float4*>(x + 4);
  float s = __uint_as_float(raw.x << 16) * a.x;
  s = fmaf(__uint_as_float(raw.x & 0xFFFF0000u), a.y, s);
  s = fmaf(__uint_as_float(raw.y << 16), a.z, s);
  s = fmaf(__uint_as_float(raw.y & 0xFFFF0000u), a.w, s);
  s = fmaf(__uint_as_float(raw.z << 16), b.x, s);
  s = fmaf(__uint_as_float(raw.z & 0xFFFF0000u), b.y, s);
  s = fmaf(__uint_as_float(raw.w << 16), b.z, s);
  return fmaf(__uint_as_float(raw.w & 0xFFFF0000u), b.w, s);
}
template <>
__device__ __forceinline__ float dot_chunk<float>(const u32x4& raw, const float* x) {
  const float4 a = *reinterpret_cast<const float4*>(x);
  float s = __uint_as_float(raw.x) * a.x;
  s = fmaf(__uint_as_float(raw.y), a.y, s);
  s = fmaf(__uint_as_float(raw.z), a.z, s);
  return fmaf(__uint_as_float(raw.w), a.w, s);
}

// Rows of one phase for this workgroup. Local row j of the job maps to a
// physical row of a row-major matrix `base` (row stride ld elements); the dot
// covers columns [col0, col0 + K). kind: 0 linear (row0 + j), 1 Q/K/V rows of
// KV head g (local index row0 + j inside the head's (G+2)*D rows), 2 gate/up
// pairs of z index row0 + j/2 (gate when j is even) in the interleaved layout.
template <typename WT>
struct Job {
  const WT* base;
  int ld, col0, K, nrows, kind, row0;
  int qd, d, nq_d, nkv_d, g;  // kind 1 mapping
  __device__ __forceinline__ int phys(int j) const {
    if (kind == 0) return row0 + j;
    if (kind == 1) {
      const int i = row0 + j;
      if (i < qd) return g * qd + i;
      if (i < qd + d) return nq_d + g * d + (i - qd);
      return nq_d + nkv_d + g * d + (i - qd - d);
    }
    const int z = row0 + (j >> 1);
    return (z / kGuGroup) * 2 * kGuGroup + ((j & 1) ? kGuGroup : 0) + z % kGuGroup;
  }
};

// Memory-wave weight staging. Each memory wave owns an LDS ring of two regions
// of kSlots slots; a slot holds one 16-byte chunk per lane (1 KB). A unit (one
// phase's rows of this wave, or one batch of LM-head rows) is copied into a
// region by direct global-to-LDS loads (lane i's 16 bytes land at slot + 16 i)
// and later read back by the same lanes for the dot products. Unit k uses
// region k & 1; after computing unit k the wave issues unit k + 2, so one unit
// is always in flight while another is consumed. The wave issues no other
// vector-memory operations, so the count of its loads issued after a unit
// tells exactly how far the vector-memory counter may lag when that unit is
// needed.
//
// Slot q of a unit covers the wave's job row i = bt * rpb + (q >> lg) and
// chunk c = lane + 64 * (q & (cpl - 1)), with cpl = 2^lg chunks per lane per
// row and rpb = kSlots >> lg rows per unit; the wave owns job rows w + 4 i.
constexpr int kSlots = 12;
constexpr int kMaxVec = 2048;  // longest GEMV input: max(hidden, G * D, ffn / 8)
constexpr int kSlotBytes = kWave * 16;

typedef __attribute__((address_space(3))) void lds_void;

template <typename WT>
__device__ __forceinline__ int job_lg(const Job<WT>& jb) {
  const int nch = jb.K / (16 / (int)sizeof(WT));
  const int cpl = (nch + kWave - 1) / kWave;
  return cpl <= 1 ? 0 : cpl <= 2 ? 1 : cpl <= 4 ? 2 : 3;
}
template <typename WT>
__device__ __forceinline__ int job_rows_of_wave(const Job<WT>& jb, int w) {
  return jb.nrows > w ? (jb.nrows - w + kMemWaves - 1) / kMemWaves : 0;
}
template <typename WT>
__device__ __forceinline__ int job_units(const Job<WT>& jb, int w) {
  const int rpb = kSlots >> job_lg(jb);
  return (job_rows_of_wave(jb, w) + rpb - 1) / rpb;
}

// s_waitcnt vmcnt(n) for a wave-uniform n (loads issued after the needed ones)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define QDEC_VM(N) \
  case N:          \
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N));  \
    break;
    QDEC_VM(1) QDEC_VM(2) QDEC_VM(3) QDEC_VM(4) QDEC_VM(5) QDEC_VM(6) QDEC_VM(7) QDEC_VM(8)
    QDEC_VM(9) QDEC_VM(10) QDEC_VM(11) QDEC_VM(12) QDEC_VM(13) QDEC_VM(14) QDEC_VM(15)
#undef QDEC_VM
    default:
      __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// The two regions are distinct LDS arrays so that the compiler, which must
// wait for outstanding direct-to-LDS loads before an LDS read that may alias
// them, can tell a read of one region (or of any other LDS data) from the
// loads in flight into the other.
struct Ring {
  char* r0;    // this wave's slots in region 0
  char* r1;    // this wave's slots in region 1
  int issued;  // loads issued by this wave
  int mark0, mark1;  // `issued` right after the unit of each region was issued
};

template <int PAR, int LG, typename WT>
__device__ __forceinline__ void ring_issue_lg(Ring& rg, const Job<WT>& jb, int bt, int w, int lane) {
  constexpr int VN = 16 / sizeof(WT);
  constexpr int RPB = kSlots >> LG;
  const int nch = jb.K / VN;
  const int nrw = job_rows_of_wave(jb, w);
  char* region = PAR ? rg.r1 : rg.r0;
#pragma unroll
  for (int ii = 0; ii < RPB; ++ii) {
    const int i = bt * RPB + ii;
    if (i < nrw) {  // wave-uniform: every lane issues, so the count is exact
      const WT* rowp = jb.base + (size_t)jb.phys(w + kMemWaves * i) * jb.ld + jb.col0;
#pragma unroll
      for (int jj = 0; jj < (1 << LG); ++jj) {
        const int c = lane + kWave * jj;
        const WT* src = rowp + (size_t)(c < nch ? c : 0) * VN;
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (lds_void*)(region + (ii * (1 << LG) + jj) * kSlotBytes), 16, 0, 0);
      }
      rg.issued += 1 << LG;
    }
  }
  if (PAR)
    rg.mark1 = rg.issued;
  else
    rg.mark0 = rg.issued;
}

template <int PAR, typename WT>
__device__ __forceinline__ void ring_issue(Ring& rg, const Job<WT>& jb, int bt, int w, int lane) {
  switch (job_lg(jb)) {
    case 0: ring_issue_lg<PAR, 0>(rg, jb, bt, w, lane); break;
    case 1: ring_issue_lg<PAR, 1>(rg, jb, bt, w, lane); break;
    case 2: ring_issue_lg<PAR, 2>(rg, jb, bt, w, lane); break;
    default: ring_issue_lg<PAR, 3>(rg, jb, bt, w, lane); break;
  }
}

template <int PAR>
__device__ __forceinline__ void ring_wait(const Ring& rg) {
  wait_vm(rg.issued - (PAR ? rg.mark1 : rg.mark0));
}

// Dot products of a unit whose loads are complete (ring_wait): f(j, value)
// for every job row j of this wave in batch bt (value wave-reduced and
// wave-uniform; called by all lanes).
template <int PAR, int LG, typename WT, typename Fn>
__device__ __forceinline__ void ring_dot_lg(const Ring& rg, const Job<WT>& jb, int bt, const float* x, int w, int lane,
                                            Fn f) {
  constexpr int VN = 16 / sizeof(WT);
  constexpr int RPB = kSlots >> LG;
  const int nch = jb.K / VN;
  const int nrw = job_rows_of_wave(jb, w);
  const char* region = PAR ? rg.r1 : rg.r0;
  // this lane's input chunks are the same for every row of the unit
  float xv[1 << LG][VN];
#pragma unroll
  for (int jj = 0; jj < (1 << LG); ++jj) {
    const int c = lane + kWave * jj;
#pragma unroll
    for (int e = 0; e < VN; e += 4) {
      const float4 t = c < nch ? *reinterpret_cast<const float4*>(x + c * VN + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[jj][e] = t.x; xv[jj][e + 1] = t.y; xv[jj][e + 2] = t.z; xv[jj][e + 3] = t.w;
    }
  }
#pragma unroll
  for (int ii = 0; ii < RPB; ++ii) {
    if (bt * RPB + ii < nrw) {
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < (1 << LG); ++jj) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(region + (ii * (1 << LG) + jj) * kSlotBytes + lane * 16);
        acc += dot_chunk<WT>(raw, xv[jj]);
      }
      f(w + kMemWaves * (bt * RPB + ii), wave_sum(acc));
    }
  }
}

template <int PAR, typename WT, typename Fn>
__device__ __forceinline__ void ring_dot(const Ring& rg, const Job<WT>& jb, int bt, const float* x, int w, int lane,
                                         Fn f) {
  switch (job_lg(jb)) {
    case 0: ring_dot_lg<PAR, 0>(rg, jb, bt, x, w, lane, f); break;
    case 1: ring_dot_lg<PAR, 1>(rg, jb, bt, x, w, lane, f); break;
    case 2: ring_dot_lg<PAR, 2>(rg, jb, bt, x, w, lane, f); break;
    default: ring_dot_lg<PAR, 3>(rg, jb, bt, x, w, lane, f); break;
  }
}

// ---------------------------------------------------------------- attention

// K/V of cached position u for KV head g, DPL floats at dims part*DPL.. ;
// `fresh` positions were written earlier in this launch by another CU and are
// read with device-scope loads.
template <int DPL>
__device__ __forceinline__ void load_kv(const DecParams& p, int l, int g, int u, int part, bool fresh, float* kv,
                                        float* vv) {
  const float* page = reinterpret_cast<const float*>(p.page_table[u / kPage]);
  Dims dd{p.L, 0, 0, p.NKV, DPL * 8, 0, 0, 0.f};
  const float* kp = page + page_offset(dd, l, 0, g, u % kPage) + part * DPL;
  const float* vp = page + page_offset(dd, l, 1, g, u % kPage) + part * DPL;
  if (!fresh) {
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(kp + i);
      kv[i] = a.x; kv[i + 1] = a.y; kv[i + 2] = a.z; kv[i + 3] = a.w;
      const float4 c = *reinterpret_cast<const float4*>(vp + i);
      vv[i] = c.x; vv[i + 1] = c.y; vv[i + 2] = c.z; vv[i + 3] = c.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DPL; i += 2) {
      const u64 a = get(reinterpret_cast<const u64*>(kp + i));
      kv[i] = __uint_as_float((unsigned)a); kv[i + 1] = __uint_as_float((unsigned)(a >> 32));
      const u64 c = get(reinterpret_cast<const u64*>(vp + i));
      vv[i] = __uint_as_float((unsigned)c); vv[i + 1] = __uint_as_float((unsigned)(c >> 32));
    }
  }
}

// Online-softmax attention of the G query heads of KV head g over the keys
// [u0, u0 + n_cached) of the cache plus (if with_cur) the current token held
// in LDS, run by the exchange waves. Lane layout: key slot = lane / 8 (8 keys
// per wave per iteration), part = lane % 8 owns DPL = D/8 dims. Result per head
// (combined over the waves): M, Lsum and the unnormalised O, written to
// res[h * (D + 2) + {0, 1, 2..}]. The first two iterations' K/V come from
// prefetch().
template <int D, int G>
struct Attn {
  static constexpr int DPL = D / 8;
  static constexpr int kPerIt = kExWaves * 8;  // keys per iteration
  float kv0[DPL], vv0[DPL], kv1[DPL], vv1[DPL];

  __device__ __forceinline__ void prefetch(const DecParams& p, int l, int g, int u0, int n_cached, int ew, int lane) {
    const int slot = lane / 8, part = lane % 8;
    const int k0 = ew * 8 + slot, k1 = k0 + kPerIt;
    if (k0 < n_cached) load_kv<DPL>(p, l, g, u0 + k0, part, u0 + k0 >= p.pos0, kv0, vv0);
    if (k1 < n_cached) load_kv<DPL>(p, l, g, u0 + k1, part, u0 + k1 >= p.pos0, kv1, vv1);
  }

  __device__ __forceinline__ void step(const float* q_l, const float* k_l, const float* v_l, const float* kv,
                                       const float* vv, int kidx, int n_cached, int n_keys, int part, float* m,
                                       float* ls, float (*acc)[DPL]) {
    const bool valid = kidx < n_keys;
    float kk[DPL], vvv[DPL];
    if (kidx >= n_cached && valid) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        kk[i] = k_l[part * DPL + i];
        vvv[i] = v_l[part * DPL + i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        kk[i] = valid ? kv[i] : 0.f;
        vvv[i] = valid ? vv[i] : 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; i += 4) {
        const float4 q = *reinterpret_cast<const float4*>(q_l + h * D + part * DPL + i);
        sc = fmaf(q.x, kk[i], sc);
        sc = fmaf(q.y, kk[i + 1], sc);
        sc = fmaf(q.z, kk[i + 2], sc);
        sc = fmaf(q.w, kk[i + 3], sc);
      }
      // sum over the 8 parts of a key (quad steps, then the two quads of the 8)
      sc += dpp<kDppXor1>(sc);
      sc += dpp<kDppXor2>(sc);
      sc += dpp<kDppHalfMirror>(sc);
      if (!valid) sc = -INFINITY;
      // max over the 8 keys of the wave (values are uniform within each 8 lanes)
      float mx = fmaxf(sc, dpp<kDppMirror>(sc));
      mx = max32(max16(mx));
      const float mn = fmaxf(m[h], mx);
      if (mn == -INFINITY) continue;  // nothing valid seen yet by this wave (wave-uniform)
      const float alpha = expf(m[h] - mn);
      const float pr = valid ? expf(sc - mn) : 0.f;
      float ps = pr + dpp<kDppMirror>(pr);
      ps = sum32(sum16(ps));
      ls[h] = ls[h] * alpha + ps;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[h][i] = fmaf(pr, vvv[i], acc[h][i] * alpha);
      m[h] = mn;
    }
  }

  // All threads call; only `act` threads compute. q_l: [G][D] (scaled), k_l,
  // v_l: [D] current token; wbuf scratch: 2 * kExWaves * G + kExWaves * G * D.
  __device__ __forceinline__ void run(bool act, const DecParams& p, int l, int g, int u0, int n_cached,
                                      bool with_cur, const float* q_l, const float* k_l, const float* v_l,
                                      float* wbuf, float* res, int ew, int lane, int et) {
    float* wm = wbuf;                     // [kExWaves][G]
    float* wl = wm + kExWaves * G;        // [kExWaves][G]
    float* wo = wl + kExWaves * G;        // [kExWaves][G][D]
    if (act) {
      const int slot = lane / 8, part = lane % 8;
      float m[G], ls[G], acc[G][DPL];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        ls[h] = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[h][i] = 0.f;
      }
      const int n_keys = n_cached + (with_cur ? 1 : 0);
      for (int base = 0; base < n_keys; base += 2 * kPerIt) {
        const int ka = base + ew * 8 + slot;
        step(q_l, k_l, v_l, kv0, vv0, ka, n_cached, n_keys, part, m, ls, acc);
        const int kn0 = ka + 2 * kPerIt;
        if (kn0 < n_cached) load_kv<DPL>(p, l, g, u0 + kn0, part, u0 + kn0 >= p.pos0, kv0, vv0);
        const int kb = ka + kPerIt;
        if (base + kPerIt < n_keys) step(q_l, k_l, v_l, kv1, vv1, kb, n_cached, n_keys, part, m, ls, acc);
        const int kn1 = kb + 2 * kPerIt;
        if (kn1 < n_cached) load_kv<DPL>(p, l, g, u0 + kn1, part, u0 + kn1 >= p.pos0, kv1, vv1);
      }
      // sum the 8 key slots of the wave (same running max within the wave)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          float v = acc[h][i];
          v += dpp<kDppXor8>(v);  // same part of the other key slot in the row
          v = sum32(sum16(v));
          acc[h][i] = v;
        }
      if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int i = 0; i < DPL; ++i) wo[(ew * G + h) * D + part * DPL + i] = acc[h][i];
      }
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          wm[ew * G + h] = m[h];
          wl[ew * G + h] = ls[h];
        }
      }
    }
    __syncthreads();
    if (act) {
      for (int idx = et; idx < G * (D + 2); idx += kEx) {
        const int h = idx / (D + 2), e = idx % (D + 2);
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < kExWaves; ++w2) M = fmaxf(M, wm[w2 * G + h]);
        float v = 0.f;
        if (e == 0) {
          v = M;
        } else {
#pragma unroll
          for (int w2 = 0; w2 < kExWaves; ++w2) {
            const float mw = wm[w2 * G + h];
            const float f = (mw == -INFINITY) ? 0.f : expf(mw - M);
            v = fmaf(f, e == 1 ? wl[w2 * G + h] : wo[(w2 * G + h) * D + (e - 2)], v);
          }
        }
        res[idx] = v;
      }
    }
    __syncthreads();
  }
};

// ------------------------------------------------------------------- kernel

using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

template <typename WT, int D, int G, int NE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecParams p) {
  extern __shared__ float sm[];
  constexpr int QD = G * D, GW = (G + 2) * D;
  float* xres = sm + p.lds_x;      // residual stream [H], identical in every workgroup
  // GEMV input (normalised x, o_g or z slice): its own LDS array, read while
  // weight loads into the rings are in flight
  __shared__ __attribute__((aligned(16))) float xn[kMaxVec];
  float* stage = sm + p.lds_stage; // raw q/k/v, split partials, argmax keys
  float* att = sm + p.lds_att;     // q_l [G][D] | k_l [D] | v_l [D] | res [G][D+2] | wave scratch
  float* red = sm + p.lds_red;     // [64] reductions
  float* rbuf = sm + p.lds_rbuf;   // [64] dot results of the memory waves
  float* lgb = sm + p.lds_lgb;     // this workgroup's logits of one step
  float* q_l = att;
  float* k_l = q_l + QD;
  float* v_l = k_l + D;
  float* ares = v_l + D;
  float* wscr = ares + G * (D + 2);

  const int tid0 = threadIdx.x;
  const int lane0 = tid0 % kWave;
  const int wave0 = __builtin_amdgcn_readfirstlane(tid0 / kWave);
  const bool mem = wave0 < kMemWaves;  // wave-uniform role
  const bool ex = !mem;
  const int b = blockIdx.x, nb = gridDim.x;
  const int X = b % kGroups, r = b / kGroups, R = p.R;
  const int H = p.H, F = p.F, NKV = p.NKV, NQ = p.NQ, L = p.L;
  const int FS = F / kGroups;
  const bool has_att = X < NKV;
  const WT* embed = (const WT*)p.embed;

  // this workgroup's row ranges (fixed for all layers)
  int a0_, a1_, c0_, c1_, z0_, z1_, e0_, e1_, h0_, h1_;
  split(GW, R, r, a0_, a1_);
  split(H, R, r, c0_, c1_);
  split(FS, R, r, z0_, z1_);
  split(H, R, r, e0_, e1_);
  split(p.V, nb, b, h0_, h1_);

  auto WL = [&](int l) { return (const WT*)p.wbuf + (size_t)l * p.layer_elems; };
  // weight units of one step, in the order the memory waves consume them:
  // with attention A, C, D, E per layer, else D, E per layer; then LM-head batches
  const int per_layer = has_att ? 4 : 2;
  const int n_layer_units = per_layer * L;
  auto unit_job = [&](int k, int a0, int a1, int c0, int c1, int z0, int z1, int e0, int e1, int h0, int h1,
                      int& bt) __attribute__((always_inline)) {
    bt = 0;
    if (k >= n_layer_units) {
      bt = k - n_layer_units;
      return Job<WT>{embed, H, 0, H, h1 - h0, 0, h0, 0, 0, 0, 0, 0};
    }
    const int l = k / per_layer;
    int t = k % per_layer;
    if (!has_att) t += 2;
    if (t == 0) return Job<WT>{WL(l), H, 0, H, a1 - a0, 1, a0, QD, D, NQ * D, NKV * D, X};
    if (t == 1) return Job<WT>{WL(l) + p.off_o, NQ * D, X * QD, QD, c1 - c0, 0, c0, 0, 0, 0, 0, 0};
    if (t == 2) return Job<WT>{WL(l) + p.off_gu, H, 0, H, 2 * (z1 - z0), 2, X * FS + z0, 0, 0, 0, 0, 0};
    return Job<WT>{WL(l) + p.off_d, F, X * FS, FS, e1 - e0, 0, e0, 0, 0, 0, 0, 0};
  };

  __shared__ __attribute__((aligned(16))) char ring0[kMemWaves * kSlots * kSlotBytes];
  __shared__ __attribute__((aligned(16))) char ring1[kMemWaves * kSlots * kSlotBytes];
  const int rw = mem ? wave0 : 0;
  Ring rg{ring0 + rw * kSlots * kSlotBytes, ring1 + rw * kSlots * kSlotBytes, 0, 0, 0};
  int token = p.token_dev ? p.token_dev[0] : p.token;
  token = token < 0 ? 0 : (token >= p.V ? p.V - 1 : token);

  for (int step = 0; step < p.nsteps; ++step) {
    const int pos = p.pos0 + step;
    const int n_hist = pos;  // cached positions 0 .. pos-1
    int n_units = 0;
    {
      // Index bases made opaque per iteration: keeps per-row address arithmetic
      // from being hoisted out of the loops and held in registers.
      int tid = tid0, lane = lane0, wave = wave0, a0 = a0_, a1 = a1_, c0 = c0_, c1 = c1_, z0 = z0_, z1 = z1_,
          e0 = e0_, e1 = e1_, h0 = h0_, h1 = h1_;
      asm volatile("" : "+v"(tid), "+v"(lane));
      asm volatile("" : "+s"(wave), "+s"(a0), "+s"(a1), "+s"(c0), "+s"(c1), "+s"(z0), "+s"(z1));
      asm volatile("" : "+s"(e0), "+s"(e1), "+s"(h0), "+s"(h1));
      TRACE(step, 0);
      if (mem) {
        const Job<WT> jh{embed, H, 0, H, h1 - h0, 0, h0, 0, 0, 0, 0, 0};
        n_units = n_layer_units + job_units(jh, wave);
        int bt;
        const Job<WT> j0 = unit_job(0, a0, a1, c0, c1, z0, z1, e0, e1, h0, h1, bt);
        ring_issue<0>(rg, j0, bt, wave, lane);
        const Job<WT> j1 = unit_job(1, a0, a1, c0, c1, z0, z1, e0, e1, h0, h1, bt);
        ring_issue<1>(rg, j1, bt, wave, lane);
      } else {
        for (int i = tid - kExBase; i < H; i += kEx) xres[i] = wload(embed, (size_t)token * H + i);
      }
      __syncthreads();
    }

    // Consume unit k (its region is PAR = k & 1), then issue unit k + 2 into that region.
    auto unit = [&](auto par_tag, int k, const float* x, auto f, int ti = -1) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value;
      (void)ti;
      TRACEM(step, ti);
      int lane = lane0, wave = wave0, a0 = a0_, a1 = a1_, c0 = c0_, c1 = c1_, z0 = z0_, z1 = z1_, e0 = e0_,
          e1 = e1_, h0 = h0_, h1 = h1_;
      asm volatile("" : "+v"(lane));
      asm volatile("" : "+s"(wave), "+s"(a0), "+s"(a1), "+s"(c0), "+s"(c1), "+s"(z0), "+s"(z1));
      asm volatile("" : "+s"(e0), "+s"(e1), "+s"(h0), "+s"(h1));
      int bt;
      const Job<WT> j = unit_job(k, a0, a1, c0, c1, z0, z1, e0, e1, h0, h1, bt);
      ring_wait<PAR>(rg);
      TRACEM(step, ti < 0 ? -1 : ti + 1);
      ring_dot<PAR>(rg, j, bt, x, wave, lane, f);
      TRACEM(step, ti < 0 ? -1 : ti + 2);
      if (k + 2 < n_units) {
        int bt2;
        const Job<WT> j2 = unit_job(k + 2, a0, a1, c0, c1, z0, z1, e0, e1, h0, h1, bt2);
        ring_issue<PAR>(rg, j2, bt2, wave, lane);
      }
      TRACEM(step, ti < 0 ? -1 : ti + 3);
    };

    // attention mode for this step
    const bool whole = n_hist <= p.whole_max;
    int nsplit = 1;
    if (!whole) nsplit = min(p.nsplit_max, (n_hist + p.whole_max - 1) / p.whole_max);

    for (int l = 0; l < L; ++l) {
      int tid = tid0, lane = lane0, wave = wave0, a0 = a0_, a1 = a1_, c0 = c0_, c1 = c1_, z0 = z0_, z1 = z1_,
          e0 = e0_, e1 = e1_;
      asm volatile("" : "+v"(tid), "+v"(lane));
      asm volatile("" : "+s"(wave), "+s"(a0), "+s"(a1), "+s"(c0), "+s"(c1), "+s"(z0), "+s"(z1));
      asm volatile("" : "+s"(e0), "+s"(e1));
      const int et = tid - kExBase;  // exchange thread index (meaningful when ex)
      const int ew = wave - kMemWaves;
      const int ku = l * per_layer;  // this layer's first unit
      const int gl = step * L + l;
      const int par = gl & 1, ppar = par ^ 1;
      const unsigned tg = p.tag0 + (unsigned)((step * (L + 1) + l) * kTagSlots);
      const unsigned tgp = tg - kTagSlots;  // layer l-1 of this step
      u64* Lq = p.ll + p.o_q + ((size_t)par * NKV + X) * GW;
      u64* La = p.ll + p.o_att + ((size_t)par * NKV + X) * R * G * (D + 2);
      u64* Lo = p.ll + p.o_o + (size_t)par * NKV * H;
      u64* Lz = p.ll + p.o_z + ((size_t)par * kGroups + X) * FS;
      u64* Lx = p.ll + p.o_x + (size_t)par * kGroups * H;
      const u64* Lx_prev = p.ll + p.o_x + (size_t)ppar * kGroups * H;
      const float* nrm = p.nbuf + (size_t)l * p.norm_elems;
      const float *g_in = nrm, *g_post = nrm + H, *g_q = nrm + 2 * H, *g_k = nrm + 2 * H + D;
      auto to_rbuf = [&](int j, float v) __attribute__((always_inline)) {
        if (lane == 0) rbuf[j] = v;
      };

      TRACE(step, 1 + l * 12 + 0);
      if (l > 0) {
        if (!gather_sum<NE>(ex, Lx_prev, kGroups, H, tgp + PH_X, xres, et)) {
          fail_launch(p.err, tid);
          return;
        }
      }
      TRACE(step, 1 + l * 12 + 1);
      if (has_att) {
        // ---------------- A
        int u0 = 0, n_cached = n_hist;
        const bool att_rank = whole || r < nsplit;
        if (!whole) {
          int su, se;
          split(n_hist, nsplit, r, su, se);
          u0 = su;
          n_cached = se - su;
        }
        rms_norm(ex, xres, g_in, H, p.eps, xn, red, tid, et);
        Attn<D, G> at;
        if (mem) {
          unit(P0{}, ku + 0, xn, to_rbuf, 200 + 4 * l);
        } else if (att_rank) {
          // cached K/V of the first two iterations do not depend on this token:
          // their loads overlap the wait for the group's Q/K/V rows
          at.prefetch(p, l, X, u0, n_cached, ew, lane);
        }
        __syncthreads();
        if (ex)
          for (int i = et; i < a1 - a0; i += kEx) put(Lq + a0 + i, rbuf[i], tg + PH_Q);
        TRACE(step, 1 + l * 12 + 2);

        // ---------------- B
        if (!gather_vec<(GW + kEx - 1) / kEx>(ex, Lq, GW, tg + PH_Q, stage, et)) {
          fail_launch(p.err, tid);
          return;
        }
        TRACE(step, 1 + l * 12 + 3);
        if (ex) {
          // per-head RMSNorm + RoPE: head vectors 0..G-1 are q, G is k; v copied
          for (int hv = ew; hv <= G + 1; hv += kExWaves) {
            const float* src = stage + hv * D;
            if (hv == G + 1) {
              for (int i = lane; i < D; i += kWave) v_l[i] = src[i];
              continue;
            }
            const float* gg = hv < G ? g_q : g_k;
            constexpr int half = D / 2;
            float va = 0.f, vb = 0.f;
            if (lane < half) {
              va = src[lane];
              vb = src[lane + half];
            }
            const float ss = wave_sum(va * va + vb * vb);
            const float inv = 1.f / sqrtf(ss / (float)D + p.eps);
            if (lane < half) {
              va = va * inv * gg[lane];
              vb = vb * inv * gg[lane + half];
              const float c = p.rope_cos[(size_t)pos * half + lane], sn = p.rope_sin[(size_t)pos * half + lane];
              const float ra = va * c - vb * sn, rb = vb * c + va * sn;
              if (hv < G) {
                q_l[hv * D + lane] = ra * p.scale;
                q_l[hv * D + lane + half] = rb * p.scale;
              } else {
                k_l[lane] = ra;
                k_l[lane + half] = rb;
              }
            }
          }
        }
        __syncthreads();
        if (ex && r == 0) {  // append K and V at pos (write-through; completion awaited before phase C ends)
          float* page = reinterpret_cast<float*>(p.page_table[pos / kPage]);
          Dims dd{L, 0, 0, NKV, D, 0, 0, 0.f};
          for (int i = et; i < 2 * D; i += kEx) {
            const int sel = i / D, d = i % D;
            __hip_atomic_store(page + page_offset(dd, l, sel, X, pos % kPage) + d, sel ? v_l[d] : k_l[d],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        at.run(ex && att_rank, p, l, X, u0, n_cached, whole || r == nsplit - 1, q_l, k_l, v_l, wscr, ares, ew,
               lane, et);
        TRACE(step, 1 + l * 12 + 4);
        // ---------------- C
        if (whole) {
          if (ex) {
            for (int idx = et; idx < QD; idx += kEx) {
              const int h = idx / D, d = idx % D;
              xn[idx] = ares[h * (D + 2) + 2 + d] / ares[h * (D + 2) + 1];
            }
            if (r == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // KV append stores complete
          }
          __syncthreads();
        } else {
          if (ex && r < nsplit) {
            for (int idx = et; idx < G * (D + 2); idx += kEx)
              put(La + (size_t)r * G * (D + 2) + idx, ares[idx], tg + PH_ATT);
          }
          if (ex && r == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // KV append stores complete
          if (!gather_any(ex, La, nsplit * G * (D + 2), tg + PH_ATT, stage, et)) {
            fail_launch(p.err, tid);
            return;
          }
          if (ex) {
            for (int idx = et; idx < QD; idx += kEx) {
              const int h = idx / D, d = idx % D;
              float M = -INFINITY;
              for (int s = 0; s < nsplit; ++s) M = fmaxf(M, stage[(s * G + h) * (D + 2)]);
              float o = 0.f, lt = 0.f;
              for (int s = 0; s < nsplit; ++s) {
                const float* ps = stage + (s * G + h) * (D + 2);
                const float f = (ps[0] == -INFINITY) ? 0.f : expf(ps[0] - M);
                o = fmaf(f, ps[2 + d], o);
                lt = fmaf(f, ps[1], lt);
              }
              xn[idx] = o / lt;
            }
          }
          __syncthreads();
        }
        TRACE(step, 1 + l * 12 + 5);
        if (mem) unit(P1{}, ku + 1, xn, to_rbuf);
        __syncthreads();
        if (ex)
          for (int i = et; i < c1 - c0; i += kEx) put(Lo + (size_t)X * H + c0 + i, rbuf[i], tg + PH_O);
      }

      // ---------------- D
      TRACE(step, 1 + l * 12 + 6);
      if (!gather_sum<NE>(ex, Lo, NKV, H, tg + PH_O, xres, et)) {
        fail_launch(p.err, tid);
        return;
      }
      TRACE(step, 1 + l * 12 + 7);
      rms_norm(ex, xres, g_post, H, p.eps, xn, red, tid, et);
      if (mem) unit(P0{}, ku + per_layer - 2, xn, to_rbuf);
      __syncthreads();
      if (ex) {
        for (int i = et; i < z1 - z0; i += kEx) {
          const float gt = rbuf[2 * i], up = rbuf[2 * i + 1];
          put(Lz + z0 + i, gt / (1.f + expf(-gt)) * up, tg + PH_Z);
        }
      }
      TRACE(step, 1 + l * 12 + 8);

      // ---------------- E
      if (!gather_any(ex, Lz, FS, tg + PH_Z, xn, et)) {
        fail_launch(p.err, tid);
        return;
      }
      TRACE(step, 1 + l * 12 + 9);
      if (mem) unit(P1{}, ku + per_layer - 1, xn, to_rbuf);
      __syncthreads();
      if (ex)
        for (int i = et; i < e1 - e0; i += kEx) put(Lx + (size_t)X * H + e0 + i, rbuf[i], tg + PH_X);
      TRACE(step, 1 + l * 12 + 10);
    }

    // ---------------- final RMSNorm + tied LM head + greedy argmax
    {
      int tid = tid0, lane = lane0, wave = wave0, h0 = h0_, h1 = h1_;
      asm volatile("" : "+v"(tid), "+v"(lane));
      asm volatile("" : "+s"(wave), "+s"(h0), "+s"(h1));
      const int et = tid - kExBase;
      const int gl_last = step * L + L - 1;
      const unsigned tgl = p.tag0 + (unsigned)((step * (L + 1) + L - 1) * kTagSlots);
      const u64* Lx_last = p.ll + p.o_x + (size_t)(gl_last & 1) * kGroups * H;
      if (!gather_sum<NE>(ex, Lx_last, kGroups, H, tgl + PH_X, xres, et)) {
        fail_launch(p.err, tid);
        return;
      }
      TRACE(step, 400);
      rms_norm(ex, xres, p.final_norm, H, p.eps, xn, red, tid, et);
      u64* bk = reinterpret_cast<u64*>(red);
      if (mem) {
        u64 best = 0ull;
        auto logit = [&](int j, float v) __attribute__((always_inline)) {
          if (lane == 0) lgb[j] = v;
          const u64 key = argmax_key(v, h0 + j);
          best = key > best ? key : best;
        };
        // head units start at an even index: regions alternate 0, 1, 0, ...
        for (int k = n_layer_units; k < n_units; k += 2) {
          const int hu = k - n_layer_units;
          unit(P0{}, k, xn, logit, hu < 16 ? 320 + 4 * hu : -1);
          if (k + 1 < n_units) unit(P1{}, k + 1, xn, logit, hu + 1 < 16 ? 320 + 4 * (hu + 1) : -1);
        }
        if (lane == 0) bk[wave] = best;
      }
      __syncthreads();
      TRACE(step, 401);
      const int kpar = step & 1;
      u64* Lk = p.ll + p.o_key + (size_t)kpar * 2 * nb;
      const unsigned ktag = p.tag0 + (unsigned)((step * (L + 1) + L) * kTagSlots) + PH_KEY;
      if (ex) {
        if (p.logits) {
          float* lg = p.logits + (size_t)step * p.V;
          for (int j = et; j < h1 - h0; j += kEx) lg[h0 + j] = lgb[j];
        }
        if (et == 0) {
          u64 b2 = bk[0];
          for (int i = 1; i < kMemWaves; ++i) b2 = bk[i] > b2 ? bk[i] : b2;
          put(Lk + 2 * b, __uint_as_float((unsigned)(b2 >> 32)), ktag);
          put(Lk + 2 * b + 1, __uint_as_float((unsigned)b2), ktag);
        }
      }
      const bool need = (step + 1 < p.nsteps) || b == 0;
      if (need) {
        float* kw = stage;
        if (!gather_any(ex, Lk, 2 * nb, ktag, kw, et)) {
          fail_launch(p.err, tid);
          return;
        }
        TRACE(step, 402);
        u64 b3 = 0ull;
        for (int i = 0; i < nb; ++i) {
          const u64 k = ((u64)__float_as_uint(kw[2 * i]) << 32) | (u64)__float_as_uint(kw[2 * i + 1]);
          b3 = k > b3 ? k : b3;
        }
        token = (int)(0xFFFFFFFFu - (uint32_t)(b3 & 0xFFFFFFFFull));
        if (b == 0 && et == 0) p.tokens_out[step] = token;
        __syncthreads();
      }
    }
  }
}

// Dynamic LDS layout (floats): x[H] | xn[max(H, QD, FS)] | stage | att | red[64] | rbuf[64] | lgb
struct Layout {
  int x, xn, stage, att, red, rbuf, lgb, ring, total;
};
Layout layout(const Dims& d, int R, int nsplit_max, int nb) {
  const int G = d.NQ / d.NKV;
  const int QD = G * d.D, GW = (G + 2) * d.D;
  const int xn = 0;  // the GEMV input vector is a static LDS array of the kernel
  int stage = std::max(GW, nsplit_max * G * (d.D + 2));
  stage = std::max(stage, 2 * nb);  // argmax keys
  const int att = QD + 2 * d.D + G * (d.D + 2) + 2 * kExWaves * G + kExWaves * G * d.D;
  (void)R;
  Layout o;
  o.x = 0;
  o.xn = o.x + d.H;
  o.stage = o.xn + xn;
  o.att = o.stage + stage;
  o.red = o.att + att;
  o.rbuf = o.red + 64;
  o.lgb = o.rbuf + 64;
  o.ring = 0;  // the rings are static LDS arrays of the kernel
  o.total = o.lgb + (d.V + nb - 1) / nb;
  return o;
}

const void* kernel_for(bool bf16, const Dims& d) {
  const int G = d.NQ / d.NKV;
  const int NE = (d.H + kEx - 1) / kEx;
#define QDEC_DEC_CASE(WT, DD, GG, EE) \
  if (d.D == DD && G == GG && NE <= EE) return (const void*)decode_kernel<WT, DD, GG, EE>;
#define QDEC_DEC_ALL(WT)          \
  QDEC_DEC_CASE(WT, 128, 2, 4)    \
  QDEC_DEC_CASE(WT, 128, 1, 4)    \
  QDEC_DEC_CASE(WT, 128, 4, 4)    \
  QDEC_DEC_CASE(WT, 64, 1, 4)     \
  QDEC_DEC_CASE(WT, 64, 2, 4)     \
  QDEC_DEC_CASE(WT, 64, 4, 4)     \
  QDEC_DEC_CASE(WT, 32, 1, 4)     \
  QDEC_DEC_CASE(WT, 32, 2, 4)     \
  QDEC_DEC_CASE(WT, 32, 4, 4)
  if (bf16) {
    QDEC_DEC_ALL(uint16_t)
  } else {
    QDEC_DEC_ALL(float)
  }
#undef QDEC_DEC_ALL
#undef QDEC_DEC_CASE
  return nullptr;
}

}  // namespace

size_t dec_lds_bytes(const Dims& d, int R, int nsplit_max) {
  return (size_t)layout(d, R, nsplit_max, R * kGroups).total * sizeof(float);
}

size_t dec_words(const Dims& d, int nb, int nsplit_max, DecOffsets* off) {
  const int G = d.NQ / d.NKV;
  const int GW = (G + 2) * d.D;
  const int R = nb / kGroups;
  (void)nsplit_max;
  size_t o = 0;
  off->q = o; o += 2 * (size_t)d.NKV * GW;
  off->att = o; o += 2 * (size_t)d.NKV * R * G * (d.D + 2);
  off->o = o; o += 2 * (size_t)d.NKV * d.H;
  off->z = o; o += 2 * (size_t)kGroups * (d.F / kGroups);
  off->x = o; o += 2 * (size_t)kGroups * d.H;
  off->key = o; o += 2 * 2 * (size_t)nb;
  return o;
}

unsigned dec_tags_per_step(const Dims& d) { return (unsigned)((d.L + 1) * kTagSlots); }

// Every layer phase of a workgroup must fit one ring region per memory wave:
// (rows per wave) * (chunks per lane per row) <= kSlots.
bool dec_fits(bool bf16, const Dims& d, int nblocks) {
  const int R = nblocks / kGroups;
  const int VN = bf16 ? 8 : 4;
  const int G = d.NQ / d.NKV;
  auto slots = [&](int rows_per_block, int K) {
    const int nch = K / VN;
    const int cpl = (nch + kWave - 1) / kWave;
    if (cpl > 8) return 1 << 20;
    const int cplp = cpl <= 1 ? 1 : cpl <= 2 ? 2 : cpl <= 4 ? 4 : 8;
    return (rows_per_block + kMemWaves - 1) / kMemWaves * cplp;
  };
  auto per = [&](int n) { return (n + R - 1) / R; };
  const int FS = d.F / kGroups;
  return slots(per((G + 2) * d.D), d.H) <= kSlots && slots(per(d.H), G * d.D) <= kSlots &&
         slots(2 * per(FS), d.H) <= kSlots && slots(per(d.H), FS) <= kSlots && slots(1, d.H) <= kSlots;
}

int dec_split_limit(const Dims& d, int nblocks) {
  const int G = d.NQ / d.NKV;
  // the partial words of all splits must fit one gather (32 words per exchange thread)
  return std::max(1, std::min(nblocks / kGroups, 32 * kEx / (G * (d.D + 2))));
}

hipError_t dec_prepare(bool bf16, const Dims& d, size_t lds, int* blocks_per_cu) {
  const void* fn = kernel_for(bf16, d);
  if (!fn) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kThreads, lds);
}

hipError_t launch_decode(const DecLaunch& a, hipStream_t st) {
  const Dims& d = a.d;
  DecParams p{};
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
  p.page_table = a.page_table;
  p.L = d.L; p.H = d.H; p.NQ = d.NQ; p.NKV = d.NKV; p.F = d.F; p.V = d.V;
  p.eps = d.eps;
  p.scale = 1.f / sqrtf((float)d.D);
  p.pos0 = a.pos;
  p.nsteps = a.nsteps;
  p.token = a.token;
  p.token_dev = a.token_dev;
  p.logits = a.logits;
  p.tokens_out = a.tokens_out;
  p.ll = a.ll;
  p.o_q = a.off.q; p.o_att = a.off.att; p.o_o = a.off.o; p.o_z = a.off.z; p.o_x = a.off.x; p.o_key = a.off.key;
  p.tag0 = a.tag0;
  p.err = a.err;
  p.R = a.nblocks / kGroups;
  p.nsplit_max = a.nsplit_max;
  p.whole_max = a.whole_max;
  const Layout lay = layout(d, p.R, a.nsplit_max, a.nblocks);
  p.lds_x = lay.x; p.lds_xn = lay.xn; p.lds_stage = lay.stage; p.lds_att = lay.att; p.lds_red = lay.red;
  p.lds_rbuf = lay.rbuf; p.lds_lgb = lay.lgb; p.lds_ring = lay.ring;
  const void* fn = kernel_for(a.bf16, d);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(fn, dim3(a.nblocks), dim3(kThreads), args, (unsigned)a.lds_bytes, st);
}

#ifdef QDEC_TRACE
extern "C" int qdec_debug_trace(unsigned long long* host, int n) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_trace), sizeof(unsigned long long) * (size_t)n, 0,
                                  hipMemcpyDeviceToHost);
}
#endif

// Fill kernel for the exchange words (used when tags are about to wrap).
__global__ void clear_words_kernel(u64* w, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) w[i] = 0ull;
}

hipError_t launch_clear_words(unsigned long long* w, size_t n, hipStream_t st) {
  clear_words_kernel<<<256, 256, 0, st>>>(w, n);
  return hipGetLastError();
}

}  // namespace qdec
