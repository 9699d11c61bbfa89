// Persistent decode for gfx950: one launch of one workgroup per CU runs one or more
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
// partials and down partials, summed in two levels: the 8 groups' partials
// of an element by its owner rank, republished inside each group, always in
// the same order, so all copies of the residual stream are bit-identical)
// and two or three inside a group.
//
// Exchange. A phase publishes each output as an 8-byte word: fp32 value in the
// low half, a tag unique to (launch, step, layer, phase) in the high half. A
// consumer polls until every word it needs carries the expected tag. Words
// that cross XCDs are device-scope relaxed atomics. Words that stay inside a
// group are plain stores read with non-temporal loads, served by the XCD's
// L2; that is correct only while the group's workgroups share one XCD, which
// the host checks with a probe launch at model creation, falling back to
// device scope for those words too (`local` = 0) when the placement differs.
// Regions are double-buffered by layer parity. Every wait has a time limit;
// on expiry the workgroup raises a host-visible error flag and stops waiting
// for the rest of the launch, so every workgroup still runs to the end and
// the launch always drains.
//
// Weights: bf16 or fp32 rows, or int8 codes (QDEC_Q8_0) whose fp16 block
// scales ride along in one extra load per weight unit; each 16-code chunk's
// partial dot is scaled by its block's scale before the lane reduction.
//
// Two roles per workgroup. A wave's vector-memory counter retires loads in
// issue order, so a load needed now cannot complete before an earlier
// prefetch. Waves 0-3 (memory waves) therefore only stream weights: each
// phase's rows are copied straight into LDS two phases ahead, and each wave
// reduces them against the phase input into per-slot partial dot products.
// Waves 4-7 (exchange waves) hold the residual stream in registers and do
// everything latency-bound: exchange polls and publishes, norm statistics,
// Q/K-norm + RoPE, attention, SiLU and the argmax. The roles meet at exactly
// two workgroup barriers per weight unit: "input ready" and "partials ready".
// The exchange waves synchronise among themselves through an LDS counter, so
// the memory waves never wait on exchange-internal steps; the one exception is
// that a memory wave issues its next prefetch only after the exchange waves
// have issued the stores that publish the unit it just reduced (those stores
// would otherwise queue behind the prefetch).
//
// RMSNorm folding: the memory waves dot the weights with x * g (gain applied,
// not yet scaled) and the exchange waves multiply each combined row by
// 1 / sqrt(mean(x^2) + eps) when they publish it.
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
constexpr int kMaxBlocks = kEx;           // one argmax key per exchange thread
constexpr u64 kWaitTicks = 200000000ull;  // 2 s of the 100 MHz realtime counter
constexpr int kTagSlots = 8;              // tags per (step, layer)
enum { PH_Q = 0, PH_ATT = 1, PH_O = 2, PH_Z = 3, PH_X = 4, PH_KEY = 5, PH_OS = 6, PH_XS = 7 };

// Weight staging. Each memory wave owns an LDS ring of two regions of kSlots
// slots; a slot holds one 16-byte chunk per lane (1 KB). A unit (one phase's
// rows of this wave, or one batch of LM-head rows) is copied into a region by
// direct global-to-LDS loads (lane i's 16 bytes land at slot + 16 i).
constexpr int kSlots = 12;
constexpr int kSlotBytes = kWave * 16;
constexpr int kMaxK = 1024;  // longest GEMV input: max(hidden, G * D, ffn / 8)
constexpr int kLayerRes = 4 * kSlots;  // row totals of one layer unit (up to 4 packed rows per slot)
constexpr int kPtabLds = kDecMaxPos / kPage;  // KV page pointers kept in LDS

__device__ __forceinline__ u64 now() { return __builtin_amdgcn_s_memrealtime(); }

#ifdef QDEC_TRACE
// Diagnostic builds only: realtime-counter stamps at phase boundaries of the
// first step of a launch, per workgroup (taken by the first exchange thread).
constexpr int kTraceN = 512;
__device__ u64 g_trace[2048 * kTraceN];
__shared__ u64 g_xtr[kTraceN];
#define TRACEC(step, l, i)                                            \
  do {                                                                \
    if ((l) >= 1 && (l) <= 3) TRACE(step, 432 + ((l) - 1) * 8 + (i)); \
  } while (0)
#define TRACEB(step, l, i)                            \
  do {                                                \
    if ((l) >= 1 && (l) <= 3) TRACE(step, 464 + ((l) - 1) * 8 + (i)); \
  } while (0)
// stamps go to LDS (xtr) and are copied out at the end, so that no store
// joins the waves' in-order memory counters
#define TRACE(step, idx)                                                               \
  do {                                                                                 \
    if ((step) == 0 && tid == kExBase && (idx) < kTraceN) g_xtr[(idx)] = now(); \
  } while (0)
#else
#define TRACE(step, idx) \
  do {                   \
  } while (0)
#define TRACEB(step, l, i) \
  do {                     \
  } while (0)
#define TRACEC(step, l, i) \
  do {                     \
  } while (0)
#endif

// Re-define per-thread indices and the parameter pointer as opaque values:
// everything derived from them is recomputed after this point instead of being
// hoisted out of the enclosing loops and held in registers.
#define QDEC_OPAQUE()                  \
  do {                                 \
    asm volatile("" : "+v"(et), "+v"(ln)); \
    asm volatile("" : "+s"(pp));       \
  } while (0)

__device__ __forceinline__ void put(u64* p, float v, unsigned tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 get(const u64* p) {
  return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(u64 w, unsigned tag) { return (unsigned)(w >> 32) == tag; }

// Exchanges inside one group use plain stores, which reach the XCD's L2, and
// non-temporal loads, which read that L2 without allocating in the CU's L1: a
// shorter round trip than device scope. This needs every workgroup of a group
// on one XCD; the host checks the placement once per model (a probe launch
// records each workgroup's XCC id) and otherwise sets `local` to 0, and these
// words then use device scope like the chip-wide ones. A reader that ever saw
// a stale value would only keep polling (tags never repeat), and the wait's
// time limit turns that into an error.
__device__ __forceinline__ void put_l(u64* p, float v, unsigned tag, bool local) {
  if (local)
    __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    put(p, v, tag);
}
// up to four group-local 8-byte loads, issued together and awaited together
__device__ __forceinline__ void get_l4(const u64* a, const u64* b, const u64* c, const u64* d, u64& x, u64& y,
                                       u64& z, u64& w, bool local) {
  if (local) {
    asm volatile(
        "global_load_dwordx2 %0, %4, off nt\n\t"
        "global_load_dwordx2 %1, %5, off nt\n\t"
        "global_load_dwordx2 %2, %6, off nt\n\t"
        "global_load_dwordx2 %3, %7, off nt\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(x), "=&v"(y), "=&v"(z), "=&v"(w)
        : "v"(a), "v"(b), "v"(c), "v"(d)
        : "memory");
  } else {
    x = get(a);
    y = get(b);
    z = get(c);
    w = get(d);
  }
}

// Global-address-space views. Pointers read back from LDS (the KV page
// table) carry no address space, and loads through them would be FLAT
// operations, which also count against the LDS counter: every LDS wait would
// then wait for those global loads too.
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) u64 gu64;
__device__ __forceinline__ u64 get_g(const gu64* p) {
  return __hip_atomic_load(const_cast<gu64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float val(u64 w) { return __uint_as_float((unsigned)w); }
// A wave-uniform 64-bit value moved to scalar registers. readfirstlane returns
// a signed int: each half is widened through unsigned, so the low half is not
// sign-extended into the high one.
__device__ __forceinline__ u64 uniform64(u64 v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return ((u64)hi << 32) | (u64)lo;
}

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
constexpr int kDppRor4 = 0x124;       // row_ror:4, lane i reads lane (i + 4) mod 16 of its row
// permlane32_swap(a, b) exchanges lanes 32-63 of a with lanes 0-31 of b;
// permlane16_swap(a, b) exchanges the odd 16-lane rows of a with the even rows
// of b. pair32(a, b): lanes 0-31 hold a[i] + a[i+32], lanes 32-63 b[i-32] + b[i].
// pair16(a, b): 16-lane rows hold [a.r0+a.r1, b.r0+b.r1, a.r2+a.r3, b.r2+b.r3].
__device__ __forceinline__ float pair32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
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
// (value of lane i) + (value of lane i ^ 16), then the same for i ^ 32: a
// 64-lane sum once the 16-lane rows are reduced
__device__ __forceinline__ float sum16(float v) { return pair16(v, v); }
__device__ __forceinline__ float sum32(float v) { return pair32(v, v); }

// Sum over the 64 lanes; every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return sum32(sum16(v));
}

// Twelve independent 64-lane sums s[0..11] reduced together: pairs of values
// share one register after each cross-lane step, so the whole batch costs
// about as much as two single sums. Slot q's total goes to dst[q].
__device__ __forceinline__ void reduce12_store(const float (&s)[kSlots], float* dst, int lane) {
  const float p0 = pair32(s[0], s[1]), p1 = pair32(s[2], s[3]);
  const float p2 = pair32(s[4], s[5]), p3 = pair32(s[6], s[7]);
  const float p4 = pair32(s[8], s[9]), p5 = pair32(s[10], s[11]);
  // 16-lane rows of q01: slots 0, 2, 1, 3; of q23: 4, 6, 5, 7; of q45: 8, 10, 9, 11
  const float q01 = pair16(p0, p1), q23 = pair16(p2, p3), q45 = pair16(p4, p5);
  const float t = q01 + dpp<kDppXor8>(q01), u = q23 + dpp<kDppXor8>(q23);
  float r8 = (lane & 8) ? u : t;  // 8-lane group g: slot (g & 1) * 4 + perm(g >> 1)
  r8 += dpp<kDppXor1>(r8);
  r8 += dpp<kDppXor2>(r8);
  r8 += dpp<kDppHalfMirror>(r8);
  float r4 = q45;  // 16-lane row w: slot 8 + perm(w)
  r4 += dpp<kDppXor1>(r4);
  r4 += dpp<kDppXor2>(r4);
  r4 += dpp<kDppHalfMirror>(r4);
  r4 += dpp<kDppMirror>(r4);
  // perm(i) = [0, 2, 1, 3][i]
  if ((lane & 7) == 0) {
    const int g = lane >> 3;
    dst[((g & 1) << 2) | (((g >> 1) & 1) << 1) | (g >> 2)] = r8;
  }
  if ((lane & 15) == 0) {
    const int w = lane >> 4;
    dst[8 + (((w & 1) << 1) | (w >> 1))] = r4;
  }
}

// Four and eight 64-lane sums, the same steps as the first slots of
// reduce12_store: slot q's total goes to dst[q].
__device__ __forceinline__ void reduce8_store(const float (&s)[8], float* dst, int lane) {
  const float p0 = pair32(s[0], s[1]), p1 = pair32(s[2], s[3]);
  const float p2 = pair32(s[4], s[5]), p3 = pair32(s[6], s[7]);
  const float q01 = pair16(p0, p1), q23 = pair16(p2, p3);
  const float t = q01 + dpp<kDppXor8>(q01), u = q23 + dpp<kDppXor8>(q23);
  float r8 = (lane & 8) ? u : t;
  r8 += dpp<kDppXor1>(r8);
  r8 += dpp<kDppXor2>(r8);
  r8 += dpp<kDppHalfMirror>(r8);
  if ((lane & 7) == 0) {
    const int g = lane >> 3;
    dst[((g & 1) << 2) | (((g >> 1) & 1) << 1) | (g >> 2)] = r8;
  }
}
__device__ __forceinline__ void reduce4_store(const float (&s)[4], float* dst, int lane) {
  const float p0 = pair32(s[0], s[1]), p1 = pair32(s[2], s[3]);
  float r = pair16(p0, p1);  // 16-lane rows: slots 0, 2, 1, 3
  r += dpp<kDppXor1>(r);
  r += dpp<kDppXor2>(r);
  r += dpp<kDppHalfMirror>(r);
  r += dpp<kDppMirror>(r);
  if ((lane & 15) == 0) {
    const int w = lane >> 4;
    dst[((w & 1) << 1) | (w >> 1)] = r;
  }
}
// Sums over the 8-lane groups of two registers a and b whose 16-lane rows
// each hold partials of one result, a's row R in lanes 8 R' .. with the sum
// of lanes i and i ^ 8 taken first: lane group G = lane / 8 ends with the
// total of row G / 2 of a (G even) or of b (G odd); lane 8 G writes it to
// dst[idx(G)].
template <typename Idx>
__device__ __forceinline__ void reduce_rows2(float a, float b, float* dst, int lane, Idx idx) {
  const float t = a + dpp<kDppXor8>(a), u = b + dpp<kDppXor8>(b);
  float r = (lane & 8) ? u : t;
  r += dpp<kDppXor1>(r);
  r += dpp<kDppXor2>(r);
  r += dpp<kDppHalfMirror>(r);
  if ((lane & 7) == 0) dst[idx(lane >> 3)] = r;
}
// Slot sums for NS slots of one unit. PK = 0: one row per slot, dst[q].
// PK = 1: lanes 0-31 and 32-63 of slot q are rows 2q and 2q + 1. PK = 2: the
// 16-lane rows of slot q are rows 4q .. 4q + 3. Row i's total goes to dst[i].
template <int PK, int NS>
__device__ __forceinline__ void reduce_store(const float (&s)[NS], float* dst, int lane) {
  if constexpr (PK == 0) {
    if constexpr (NS == 12) {
      reduce12_store(s, dst, lane);
    } else if constexpr (NS == 8) {
      reduce8_store(s, dst, lane);
    } else {
      reduce4_store(s, dst, lane);
    }
  } else if constexpr (PK == 1) {
    // v_k = pair16(s[2k], s[2k+1]): 16-lane rows hold slot 2k row 0, slot
    // 2k+1 row 0, slot 2k row 1, slot 2k+1 row 1 (each half-summed)
#pragma unroll
    for (int m = 0; m < NS / 4; ++m) {
      const float v0 = pair16(s[4 * m], s[4 * m + 1]), v1 = pair16(s[4 * m + 2], s[4 * m + 3]);
      reduce_rows2(v0, v1, dst, lane, [m](int G) {
        const int R = G >> 1, slot = 4 * m + 2 * (G & 1) + (R & 1);
        return 2 * slot + (R >> 1);
      });
    }
  } else {
#pragma unroll
    for (int m = 0; m < NS / 2; ++m)
      reduce_rows2(s[2 * m], s[2 * m + 1], dst, lane, [m](int G) { return 4 * (2 * m + (G & 1)) + (G >> 1); });
  }
}

__device__ __forceinline__ u64 argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((u64)o << 32) | (u64)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ u64 umax64(u64 a, u64 b) { return a > b ? a : b; }
__device__ __forceinline__ u64 wave_max64(u64 k) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned lo = __shfl_xor((unsigned)k, o), hi = __shfl_xor((unsigned)(k >> 32), o);
    k = umax64(k, ((u64)hi << 32) | lo);
  }
  return k;
}

// even split of n items over `parts`: [s, e) of part i
__device__ __forceinline__ void split(int n, int parts, int i, int& s, int& e) {
  const int per = (n + parts - 1) / parts;
  s = min(n, i * per);
  e = min(n, s + per);
}

// log2 of the 64-lane chunk rows a GEMV input of k elements needs (chunks of vn)
__host__ __device__ __forceinline__ int chunk_lg(int k, int vn) {
  const int nch = k / vn;
  const int cpl = (nch + kWave - 1) / kWave;
  return cpl <= 1 ? 0 : cpl <= 2 ? 1 : cpl <= 4 ? 2 : 3;
}
// log2 of the rows packed per slot for rows of k elements (chunks of vn)
// whose consecutive rows sit a fixed stride apart: as many as fit 64 lanes
// whole, at most 4
__host__ __device__ __forceinline__ int pack_lg(int k, int vn) {
  const int nch = k / vn;
  return nch <= 16 ? 2 : nch <= 32 ? 1 : 0;
}

struct DecParams {
  const void* wbuf;  // packed layers: layer l at wbuf + l * layer_elems (see LayerW)
  size_t layer_elems, off_o, off_gu, off_d;
  const float* nbuf;  // per layer: in_norm[H], post_norm[H], q_norm[D], k_norm[D]
  int norm_elems;
  const void* embed;
  const void* wscale;  // int8 weights: segmented fp16 scales, layer l at wscale + l * layer_sbytes
  size_t layer_sbytes, soff_o, soff_gu, soff_d;
  const void* escale;  // int8 weights: scales of the embedding rows
  const float* final_norm;
  const float* rope_cos;
  const float* rope_sin;
  const int64_t* page_table;
  int L, H, NQ, NKV, F, V;
  float eps, scale;  // scale: log2(e) / sqrt(head_dim), scores in base 2
  int pos0, nsteps, token;
  const int32_t* token_dev;
  float* logits;        // [nsteps, V] or null
  int32_t* tokens_out;  // [nsteps]
  u64* ll;
  size_t o_q, o_att, o_o, o_z, o_x, o_key, o_os, o_xs, o_att2;
  unsigned tag0;
  int* err;
  int local;          // 1: group-local words use workgroup scope (placement checked), 0: device scope
  int R;              // ranks per group
  int nsplit_max;     // attention splits per group
  int whole_max;      // cached positions up to which each rank runs the whole attention
  int nhu;            // LM-head units per memory wave (the largest over waves)
  int lds_stage, lds_att, lds_sbuf, lds_ptab;
};

// Workgroup-shared control words.
struct Ctl {
  int abort;                 // a wait of this workgroup timed out: skip all later waits
  int exbar;                 // arrivals at exchange-wave barriers
  int pub;                   // publishes issued (one arrival per exchange wave and weight unit)
  float red[kExWaves];       // per exchange wave: sum of squares of its residual elements
  u64 best[2][kExWaves];     // per exchange wave: argmax keys
};

template <typename WT>
__device__ __forceinline__ float wload(const WT* p, size_t i);
template <>
__device__ __forceinline__ float wload<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
template <>
__device__ __forceinline__ float wload<float>(const float* p, size_t i) { return p[i]; }

// Workgroup barrier that orders LDS only. __syncthreads() carries workgroup
// release/acquire fences, and the compiler makes a release wait for every
// outstanding direct-to-LDS load, which would drain the memory waves' weight
// prefetch at each barrier. No data crosses waves through global memory or
// through direct-to-LDS loads here (each memory wave reads only its own ring
// after waiting on its own counter), so LDS completion is all a barrier needs.
__device__ __forceinline__ void bar() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ waits
// Exchange threads only. A wait ends when every word carries the tag, when it
// runs out of time (then the workgroup's abort flag and the launch's error
// flag are raised), or at once after an abort: later values are then garbage
// and only the error flag matters.

__device__ __forceinline__ bool give_up(u64 t0, Ctl* ctl, int* err) {
  if (__hip_atomic_load(&ctl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return true;
  if (now() - t0 > kWaitTicks) {
    __hip_atomic_store(&ctl->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return true;
  }
  return false;
}

// Publish before prefetch. A CU's vector-memory requests drain roughly in
// the order they were issued, so words published just after a memory wave's
// prefetch burst reach L2 only once that burst has drained. Each exchange
// wave counts the publish of a weight unit's results in LDS right after
// issuing its stores; a memory wave issues the loads of a later unit only
// once that count covers the unit it has just reduced.
__device__ __forceinline__ void published(int lane, Ctl* ctl) {
  if (lane == 0) __hip_atomic_fetch_add(&ctl->pub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_published(int target, Ctl* ctl, int* err) {
  const u64 t0 = now();
  while (__hip_atomic_load(&ctl->pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    if (give_up(t0, ctl, err)) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Chip-wide sum of partial vectors in two levels: x[k] += sum_{q < P}
// W[q * n + e] for e = et + k * kEx < n, in part order, with the same result
// in every workgroup.
//  1. This workgroup owns elements [e0, e1) (the same range in every group).
//     The thread holding element e of that range polls its P partial words
//     (device scope: they come from every XCD), adds them to its residual
//     value in part order and publishes the sum as a group-local word of S.
//  2. Every thread then collects the sums of its elements from the owners of
//     its own group (S, served by the XCD's L2).
// A workgroup thus reads 8 bytes per owned element and partial across the
// chip instead of every partial of every element.
template <int NE>
__device__ __forceinline__ void reduce2(const u64* W, int P, int n, int e0, int e1, unsigned tag1, u64* S,
                                        unsigned tag2, float (&x)[NE], int et, Ctl* ctl, int* err, bool local) {
  static_assert(NE <= 4, "stage 2 collects up to four elements per thread");
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int e = et + k * kEx;
    if (e >= e0 && e < e1 && e < n) {
      const u64 t0 = now();
      u64 w[kGroups];
      while (true) {
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
          if (q < P) w[q] = get(W + (size_t)q * n + e);
        bool done = true;
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
          if (q < P) done = done && tagged(w[q], tag1);
        if (done || give_up(t0, ctl, err)) break;
      }
      float s = x[k];
#pragma unroll
      for (int q = 0; q < kGroups; ++q)
        if (q < P) s += val(w[q]);
      put_l(S + e, s, tag2, local);
    }
  }
  const u64 t0 = now();
  u64 w[4];
  const u64* a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = S + min(et + k * kEx, n - 1);
  while (true) {
    get_l4(a[0], a[1], a[2], a[3], w[0], w[1], w[2], w[3], local);
    bool done = true;
#pragma unroll
    for (int k = 0; k < 4; ++k) done = done && tagged(w[k], tag2);
    if (done || give_up(t0, ctl, err)) break;
  }
#pragma unroll
  for (int k = 0; k < NE; ++k)
    if (et + k * kEx < n) x[k] = val(w[k]);
}

// dst[i] = value of W[i] for i = et + j * kEx < n (n <= 4 * kEx), words of
// this group written with put_l.
__device__ __forceinline__ void gather_local(const u64* W, int n, unsigned tag, float* dst, int et, Ctl* ctl,
                                             int* err, bool local) {
  const u64 t0 = now();
  u64 w[4];
  const u64* a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = W + min(et + j * kEx, n - 1);
  while (true) {
    get_l4(a[0], a[1], a[2], a[3], w[0], w[1], w[2], w[3], local);
    bool done = true;
#pragma unroll
    for (int j = 0; j < 4; ++j) done = done && tagged(w[j], tag);
    if (done || give_up(t0, ctl, err)) break;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (et + j * kEx < n) dst[et + j * kEx] = val(w[j]);
}


// Barrier of the four exchange waves (the memory waves do not take part):
// each wave adds one arrival to an LDS counter and waits for the generation's
// total. `gen` counts arrivals expected so far (same sequence in every exchange wave).
__device__ __forceinline__ void ex_sync(int& gen, int lane, Ctl* ctl, int* err) {
  gen += kExWaves;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
  if (lane == 0) __hip_atomic_fetch_add(&ctl->exbar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const u64 t0 = now();
  while (__hip_atomic_load(&ctl->exbar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < gen) {
    if (now() - t0 > kWaitTicks) {
      __hip_atomic_store(&ctl->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// --------------------------------------------------------------- weights

template <typename WT>
__device__ __forceinline__ float dot_chunk(const u32x4& raw, const float* x);
template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(const u32x4& raw, const float* x) {
  float s = __uint_as_float(raw.x << 16) * x[0];
  s = fmaf(__uint_as_float(raw.x & 0xFFFF0000u), x[1], s);
  s = fmaf(__uint_as_float(raw.y << 16), x[2], s);
  s = fmaf(__uint_as_float(raw.y & 0xFFFF0000u), x[3], s);
  s = fmaf(__uint_as_float(raw.z << 16), x[4], s);
  s = fmaf(__uint_as_float(raw.z & 0xFFFF0000u), x[5], s);
  s = fmaf(__uint_as_float(raw.w << 16), x[6], s);
  return fmaf(__uint_as_float(raw.w & 0xFFFF0000u), x[7], s);
}
template <>
__device__ __forceinline__ float dot_chunk<float>(const u32x4& raw, const float* x) {
  float s = __uint_as_float(raw.x) * x[0];
  s = fmaf(__uint_as_float(raw.y), x[1], s);
  s = fmaf(__uint_as_float(raw.z), x[2], s);
  return fmaf(__uint_as_float(raw.w), x[3], s);
}
// 16 int8 codes (little-endian bytes of raw.x .. raw.w) times x[0..15]; each
// code converts exactly, so only the sum rounds
__device__ __forceinline__ float code(unsigned w, int byte) { return (float)((int)(w << (24 - 8 * byte)) >> 24); }
template <>
__device__ __forceinline__ float dot_chunk<int8_t>(const u32x4& raw, const float* x) {
  float s = code(raw.x, 0) * x[0];
  s = fmaf(code(raw.x, 1), x[1], s);
  s = fmaf(code(raw.x, 2), x[2], s);
  s = fmaf(code(raw.x, 3), x[3], s);
  s = fmaf(code(raw.y, 0), x[4], s);
  s = fmaf(code(raw.y, 1), x[5], s);
  s = fmaf(code(raw.y, 2), x[6], s);
  s = fmaf(code(raw.y, 3), x[7], s);
  s = fmaf(code(raw.z, 0), x[8], s);
  s = fmaf(code(raw.z, 1), x[9], s);
  s = fmaf(code(raw.z, 2), x[10], s);
  s = fmaf(code(raw.z, 3), x[11], s);
  s = fmaf(code(raw.w, 0), x[12], s);
  s = fmaf(code(raw.w, 1), x[13], s);
  s = fmaf(code(raw.w, 2), x[14], s);
  return fmaf(code(raw.w, 3), x[15], s);
}
// an IEEE half given by its bits, widened exactly
__device__ __forceinline__ float half_bits(unsigned short b) { return (float)__builtin_bit_cast(_Float16, b); }
template <typename WT>
constexpr bool kIsQ8 = std::is_same<WT, int8_t>::value;

// Rows of one phase for this workgroup. Local row j of the job maps to a
// physical row of a row-major matrix (row stride ld elements); the dot covers
// columns [col0, col0 + K). kind: 0 linear (row0 + j), 1 Q/K/V rows of KV head
// g (local index row0 + j inside the head's (G+2)*D rows), 2 gate/up pairs of
// z index row0 + j/2 (gate when j is even) in the interleaved layout.
struct Job {
  int ld, col0, K, nrows, kind, row0;
  __device__ __forceinline__ int phys(int j, int qd, int d, int nq_d, int nkv_d, int g) const {
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

typedef __attribute__((address_space(3))) void lds_void;

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

// A memory wave's ring. The two regions are distinct LDS arrays so that the
// compiler, which must wait for outstanding direct-to-LDS loads before an LDS
// read that may alias them, can tell a read of one region from the loads in
// flight into the other. The wave issues no other vector-memory operations,
// so the count of loads issued after a unit tells exactly how far the
// vector-memory counter may lag when that unit is needed.
struct Ring {
  char* r0;
  char* r1;
  int issued;        // loads issued by this wave
  int mark0, mark1;  // `issued` right after the unit of each region was issued
  char* s0;          // int8 weights: the block scales of the unit in region 0 / 1,
  char* s1;          // 64 bytes per slot (the 32 fp16 scales of the slot's row)
};

// Rows of a unit packed into one slot when they are short: with pk > 0 a
// slot holds 2^pk consecutive rows of the unit (rows `rstride` bytes apart),
// lane l serving row l >> (6 - pk) and its chunk l & (2^(6 - pk) - 1); rows
// past the unit's nrw repeat its last row.
struct Pack {
  int pk, nrw, rstride;
};

// Issue one unit into region P: slot q (q < ns) holds chunk c = lane + 64 (q & (2^lg - 1))
// (clamped to the row's last chunk) of the row starting ro(q) bytes after
// `base`, where ro(q) is lane q of `tab` (packed: of the slot's first row).
// Int8 weights (Q8) add one load of the unit's scales: lane 4 q + i (q < ns)
// brings the 16 bytes at sbase + soff, the i-th quarter of slot q's 64
// scale bytes.
template <int P, bool Q8>
__device__ __forceinline__ void issue_unit(Ring& rg, const char* base, int tab, int ns, int lg, int nchm1,
                                           int lane, const char* sbase, int soff, Pack pkd) {
  char* region = P ? rg.r1 : rg.r0;
  const int jm = (1 << lg) - 1;
  const int gl = pkd.pk ? lane >> (6 - pkd.pk) : 0;
  const int cl = pkd.pk ? lane & ((kWave >> pkd.pk) - 1) : lane;
#pragma unroll
  for (int q = 0; q < kSlots; ++q) {
    if (q < ns) {
      const int ro = __builtin_amdgcn_readlane(tab, q) + min(gl, max(pkd.nrw - 1 - (q << pkd.pk), 0)) * pkd.rstride;
      const int c = min(cl + ((q & jm) << 6), nchm1);
      __builtin_amdgcn_global_load_lds((const void*)(base + ro + c * 16), (lds_void*)(region + q * kSlotBytes), 16,
                                       0, 0);
    }
  }
  if (Q8 && ns > 0) {
    if (lane < 4 * ns)
      __builtin_amdgcn_global_load_lds((const void*)(sbase + soff), (lds_void*)(P ? rg.s1 : rg.s0), 16, 0, 0);
    ++ns;
  }
  rg.issued += ns;
  if (P)
    rg.mark1 = rg.issued;
  else
    rg.mark0 = rg.issued;
}

// Partial dot products of the unit in region P (all kSlots slots; slots past
// the unit's count hold stale data whose results nobody reads): slot q's
// chunk times this lane's input chunk (q & (2^LG - 1)), summed over the wave.
// The input must be zero past the GEMV's length up to 64 * VN * 2^LG.
template <int P, int LG, int PK, int NS, typename WT>
__device__ __forceinline__ void dot_unit(const Ring& rg, const float* xin, float* dst, int lane) {
  constexpr int VN = 16 / sizeof(WT);
  constexpr int CPL = 1 << LG;
  static_assert(PK == 0 || LG == 0, "packed rows are one chunk row long");
  const char* region = P ? rg.r1 : rg.r0;
  const int xl = PK ? lane & ((kWave >> PK) - 1) : lane;  // this lane's input chunk
  float xr[CPL][VN];
#pragma unroll
  for (int jj = 0; jj < CPL; ++jj)
#pragma unroll
    for (int e = 0; e < VN; e += 4) {
      const float4 t = *reinterpret_cast<const float4*>(xin + (xl + kWave * jj) * VN + e);
      xr[jj][e] = t.x;
      xr[jj][e + 1] = t.y;
      xr[jj][e + 2] = t.z;
      xr[jj][e + 3] = t.w;
    }
  u32x4 raw[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) raw[q] = *reinterpret_cast<const u32x4*>(region + q * kSlotBytes + lane * 16);
  float s[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) s[q] = dot_chunk<WT>(raw[q], xr[q & (CPL - 1)]);
  if constexpr (kIsQ8<WT>) {
    // one chunk row per row (LG 0): lane l holds the codes of block l / 2 of
    // its row's 32 (its packed row's 64 / 2^PK bytes of scales start at
    // 64 / 2^PK times the row's index in the slot, so the lane's scale sits
    // at 2 (l / 2) for every PK)
    static_assert(LG == 0, "int8 rows of up to 1024 inputs fill one chunk row");
    const unsigned short* sc = reinterpret_cast<const unsigned short*>(P ? rg.s1 : rg.s0) + (lane >> 1);
#pragma unroll
    for (int q = 0; q < NS; ++q) s[q] *= half_bits(sc[q * 32]);
  }
  reduce_store<PK, NS>(s, dst, lane);
}

template <int P>
__device__ __forceinline__ void ring_wait(const Ring& rg) {
  wait_vm(rg.issued - (P ? rg.mark1 : rg.mark0));
}

// Only the slots a unit fills are summed: ns rounded up to 4, 8 or 12.
template <int P, int LG, int PK, typename WT>
__device__ __forceinline__ void consume_ns(const Ring& rg, int ns, const float* xin, float* dst, int lane) {
  if (ns <= 4)
    dot_unit<P, LG, PK, 4, WT>(rg, xin, dst, lane);
  else if (ns <= 8)
    dot_unit<P, LG, PK, 8, WT>(rg, xin, dst, lane);
  else
    dot_unit<P, LG, PK, 12, WT>(rg, xin, dst, lane);
}
template <int P, typename WT>
__device__ __forceinline__ void consume_unit(const Ring& rg, int lg, int pk, int ns, const float* xin, float* dst,
                                             int lane) {
  if (pk == 2) {
    consume_ns<P, 0, 2, WT>(rg, ns, xin, dst, lane);
  } else if (pk == 1) {
    consume_ns<P, 0, 1, WT>(rg, ns, xin, dst, lane);
  } else if constexpr (kIsQ8<WT>) {
    consume_ns<P, 0, 0, WT>(rg, ns, xin, dst, lane);
  } else {
    if (lg == 0)
      consume_ns<P, 0, 0, WT>(rg, ns, xin, dst, lane);
    else if (sizeof(WT) == 2 || lg == 1)
      consume_ns<P, 1, 0, WT>(rg, ns, xin, dst, lane);
    else
      consume_ns<P, (sizeof(WT) == 2 ? 1 : 2), 0, WT>(rg, ns, xin, dst, lane);
  }
}

// ---------------------------------------------------------------- attention

// Device address of the KV page holding position u. The page pointers are
// copied to LDS at launch start (a launch covers positions < kPtabLds *
// kPage); reading them only from LDS keeps K/V loads free of any wait on
// other global loads.
__device__ __forceinline__ gfloat* page_of(const u64* ptab, int u) { return (gfloat*)ptab[u / kPage]; }

// Online-softmax attention of the G query heads of KV head g over the keys
// [u0, u0 + n_cached) of the cache plus (if with_cur) the current token held
// in LDS, one exchange wave's share. Keys are taken in blocks of KPB; wave w
// owns keys [w KPW, (w + 1) KPW) of each block.
//  - Scores: four lanes per key (lane = 4 slot + part), each holding a quarter
//    of the dims; a quad reduction gives every lane of the quad the score.
//  - Output: lanes own output dims (VD per lane) and loop over the wave's
//    keys with the probabilities broadcast from LDS, so P.V needs no
//    cross-lane reduction.
// The wave's result per head: running max, sum and unnormalised output in
// wm, wl, wo. Block 0's K/V come from prefetch(). Scores are in base 2 (q
// carries log2(e) / sqrt(D)), so the softmax uses the hardware exp2.
template <int D, int G>
struct Attn {
  static constexpr int PARTS = 4;              // lanes per key for the scores
  static constexpr int DPL = D / PARTS;        // score dims per lane
  static constexpr int KPW = kWave / PARTS;    // keys per wave per block
  static constexpr int KPB = KPW * kExWaves;   // keys per block
  static constexpr int VD = D >= kWave ? D / kWave : 1;  // output dims per lane
  static constexpr int VL = D / VD;            // lanes holding output dims
  // Lane `part` of a key holds the 4-dim chunks part, part + PARTS, part +
  // 2 PARTS, ... of that key, so the four lanes of a key read 64 contiguous
  // bytes per load. q and k rows in LDS keep each part's DPL dims together in
  // that order, padded by 4 floats after each part, so the four parts of a
  // key, read in the same instruction, sit in different banks.
  static constexpr int QS = D + 4 * PARTS;     // padded row length
  __host__ __device__ static constexpr int padi(int d) {
    return (d / 4 % PARTS) * (DPL + 4) + (d / 4 / PARTS) * 4 + d % 4;
  }
  // offset from a key's first dim of register element i (of DPL) of lane `part`
  __host__ __device__ static constexpr int kdim(int part, int i) { return (part + PARTS * (i / 4)) * 4 + i % 4; }
  float kr[DPL];      // K chunk of this lane's key
  float vr[KPW][VD];  // V of the wave's keys at this lane's dims

  // A wave's KPW keys of a block start on a page boundary (splits and blocks
  // are page aligned and KPW == kPage), so they are the slots of one KV page:
  // one wave-uniform page pointer and fixed offsets address every load. Slots
  // past the last cached key hold values of later (or never written)
  // positions of that page; they are masked out of the scores and skipped in
  // P.V. A wave whose keys all lie past the last cached one reads the last
  // cached key's page. Pages holding positions written earlier in this launch
  // (by rank 0 of the group) are read with device-scope loads.
  __device__ __forceinline__ void load_block(const DecParams& p, const u64* ptab, int l, int g, int u0, int b0,
                                             int n_cached, int ew, int lane) {
    static_assert(KPW == kPage, "a wave's keys of a block are one page");
    const int slot = lane / PARTS, part = lane % PARTS;
    const int last = n_cached > 0 ? u0 + n_cached - 1 : 0;
    const int kb = u0 + b0 + ew * KPW;  // first key of the wave, a multiple of kPage
    const gfloat* page = (const gfloat*)uniform64(ptab[min(kb, last) / kPage]);
    const size_t lk = ((size_t)(l * 2) * p.NKV + g) * kPage * D;  // layer l, K, head g, slot 0
    const size_t lv = lk + (size_t)p.NKV * kPage * D;              // V of the same head
    const gfloat* ks = page + lk + slot * D;
    const gfloat* vs = page + lv + (lane % VL) * VD;
    if (kb + KPW - 1 < p.pos0) {  // wave-uniform: every slot written before this launch
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(1))) const f32x4 gf32x4;
#pragma unroll
      for (int i = 0; i < DPL; i += 4) {
        const f32x4 a = *reinterpret_cast<gf32x4*>(ks + kdim(part, i));
        kr[i] = a.x; kr[i + 1] = a.y; kr[i + 2] = a.z; kr[i + 3] = a.w;
      }
#pragma unroll
      for (int j = 0; j < KPW; ++j)
#pragma unroll
        for (int t = 0; t < VD; ++t) vr[j][t] = vs[j * D + t];
    } else {
#pragma unroll
      for (int i = 0; i < DPL; i += 2) {
        const u64 a = get_g(reinterpret_cast<const gu64*>(ks + kdim(part, i)));
        kr[i] = __uint_as_float((unsigned)a);
        kr[i + 1] = __uint_as_float((unsigned)(a >> 32));
      }
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        if constexpr (VD % 2 == 0) {
#pragma unroll
          for (int t = 0; t < VD; t += 2) {
            const u64 a = get_g(reinterpret_cast<const gu64*>(vs + j * D + t));
            vr[j][t] = __uint_as_float((unsigned)a);
            vr[j][t + 1] = __uint_as_float((unsigned)(a >> 32));
          }
        } else {
          typedef __attribute__((address_space(1))) unsigned gu32;
#pragma unroll
          for (int t = 0; t < VD; ++t)
            vr[j][t] = __uint_as_float(__hip_atomic_load(reinterpret_cast<gu32*>(const_cast<gfloat*>(vs + j * D + t)),
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
      }
    }
  }

  __device__ __forceinline__ void prefetch(const DecParams& p, const u64* ptab, int l, int g, int u0, int n_cached,
                                           int ew, int lane) {
    load_block(p, ptab, l, g, u0, 0, n_cached, ew, lane);
  }

  // q_l: [G][D] (scaled), k_l, v_l: [D] current token; pw: this wave's
  // probabilities [G][KPW]; writes wm[ew*G + h], wl[ew*G + h], wo[(ew*G + h)*D + d].
  __device__ __forceinline__ void partial(const DecParams& p, const u64* ptab, int l, int g, int u0, int n_cached,
                                          bool with_cur, const float* q_l, const float* k_l, const float* v_l,
                                          float* pw, float* wm, float* wl, float* wo, int ew, int lane, int step = 1,
                                          int tid = 0) {
    (void)step;
    (void)tid;
    const int slot = lane / PARTS, part = lane % PARTS;
    const int n_keys = n_cached + (with_cur ? 1 : 0);
    float m[G], ls[G], o[G][VD];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      ls[h] = 0.f;
#pragma unroll
      for (int t = 0; t < VD; ++t) o[h][t] = 0.f;
    }
    for (int b0 = 0; b0 < n_keys; b0 += KPB) {
      if (b0 > 0) load_block(p, ptab, l, g, u0, b0, n_cached, ew, lane);
      const int key = b0 + ew * KPW + slot;
      if (b0 == 0) TRACEB(step, l, 1);
      // the current token's K (LDS) replaces the cached one in the four lanes
      // of its key: read straight into their K registers
      if (key == n_cached) {
#pragma unroll
        for (int i = 0; i < DPL; i += 4) {
          const float4 t4 = *reinterpret_cast<const float4*>(k_l + part * (DPL + 4) + i);
          kr[i] = t4.x;
          kr[i + 1] = t4.y;
          kr[i + 2] = t4.z;
          kr[i + 3] = t4.w;
        }
      }
      if (b0 == 0) TRACEC(step, l, 1);
      // every head's partial score in one pass over the key chunk (each head's
      // products are summed in dimension order)
      float scs[G];
#pragma unroll
      for (int h = 0; h < G; ++h) scs[h] = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; i += 4) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float4 q = *reinterpret_cast<const float4*>(q_l + h * QS + part * (DPL + 4) + i);
          scs[h] = fmaf(q.x, kr[i], scs[h]);
          scs[h] = fmaf(q.y, kr[i + 1], scs[h]);
          scs[h] = fmaf(q.z, kr[i + 2], scs[h]);
          scs[h] = fmaf(q.w, kr[i + 3], scs[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (b0 == 0 && h == 1) TRACEC(step, l, 2);
        float sc = scs[h];
        sc += dpp<kDppXor1>(sc);  // the key's four parts
        sc += dpp<kDppXor2>(sc);
        if (key >= n_keys) sc = -INFINITY;
        if (b0 == 0 && h == 0) TRACEC(step, l, 3);
        // the wave's keys sit at lanes i, i+4, i+8, i+12 of each 16-lane row
        float mx = fmaxf(sc, dpp<kDppRor4>(sc));
        mx = fmaxf(mx, dpp<kDppXor8>(mx));
        mx = max32(max16(mx));
        const float mn = fmaxf(m[h], mx);
        if (mn == -INFINITY) continue;  // no valid key seen yet by this wave (wave-uniform)
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        const float pr = key < n_keys ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
        float ps = pr + dpp<kDppRor4>(pr);
        ps += dpp<kDppXor8>(ps);
        ps = sum32(sum16(ps));
        ls[h] = ls[h] * alpha + ps;
        m[h] = mn;
#pragma unroll
        for (int t = 0; t < VD; ++t) o[h][t] *= alpha;
        if (part == 0) pw[h * KPW + slot] = pr;
      }
      if (b0 == 0) TRACEB(step, l, 6);
      // P.V: this lane's output dims over the wave's keys of the block; the
      // probabilities and the current token's V are read once, up front
      float pv[G][KPW];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < KPW; i += 4) {
          const float4 t4 = *reinterpret_cast<const float4*>(pw + h * KPW + i);
          pv[h][i] = t4.x;
          pv[h][i + 1] = t4.y;
          pv[h][i + 2] = t4.z;
          pv[h][i + 3] = t4.w;
        }
      float vcur[VD];
#pragma unroll
      for (int t = 0; t < VD; ++t) vcur[t] = v_l[(lane % VL) * VD + t];
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int kj = b0 + ew * KPW + j;  // wave-uniform
        if (kj >= n_keys) break;
        float vv[VD];
#pragma unroll
        for (int t = 0; t < VD; ++t) vv[t] = kj == n_cached ? vcur[t] : vr[j][t];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int t = 0; t < VD; ++t) o[h][t] = fmaf(pv[h][j], vv[t], o[h][t]);
      }
    }
    TRACEB(step, l, 7);
    if (lane < VL) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int t = 0; t < VD; ++t) wo[(ew * G + h) * D + lane * VD + t] = o[h][t];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        wm[ew * G + h] = m[h];
        wl[ew * G + h] = ls[h];
      }
    }
  }
};

// ------------------------------------------------------------------- kernel

template <typename WT, int D, int G, int NE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];  // 16-byte aligned: float4 rows live here
  constexpr int QD = G * D, GW = (G + 2) * D;
  constexpr int VN = 16 / sizeof(WT);
  constexpr int ES = sizeof(WT);
  constexpr bool Q8 = kIsQ8<WT>;
  constexpr int kScaleRegion = Q8 ? kSlots * 64 : 16;  // per memory wave
  // GEMV input of the current phase (x * g, o_x or z_x), zero past its length
  __shared__ __attribute__((aligned(16))) float xin[kMaxK];
  __shared__ __attribute__((aligned(16))) char ring0[kMemWaves * kSlots * kSlotBytes];
  __shared__ __attribute__((aligned(16))) char ring1[kMemWaves * kSlots * kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sring0[kMemWaves * kScaleRegion];
  __shared__ __attribute__((aligned(16))) char sring1[kMemWaves * kScaleRegion];
  __shared__ Ctl ctl;
  float* stage = sm + p.lds_stage;  // split-attention partials of all ranks
  float* att = sm + p.lds_att;      // q_l [G][D] | k_l [D] | v_l [D] | wm | wl | wo | pw
  float* sbuf = sm + p.lds_sbuf;    // per-slot partial dots [wave][unit][kSlots]
  u64* ptab = reinterpret_cast<u64*>(sm + p.lds_ptab);  // KV page pointers
  constexpr int QS = Attn<D, G>::QS;  // padded q/k row length
  float* q_l = att;                   // [G][QS]
  float* k_l = q_l + G * QS;          // [QS]
  float* v_l = k_l + QS;              // [D]
  float* wm = v_l + D;
  float* wl = wm + kExWaves * G;
  float* wo = wl + kExWaves * G;
  float* pw = wo + kExWaves * G * D;  // attention probabilities [wave][G][keys per wave]

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool mem = wave < kMemWaves;  // wave-uniform role
  const int b = blockIdx.x, nb = gridDim.x;
  const int X = b % kGroups, r = b / kGroups, R = p.R;
  const int H = p.H, F = p.F, NKV = p.NKV, NQ = p.NQ, L = p.L;
  const int FS = F / kGroups;
  const bool has_att = X < NKV;
  const int per_layer = has_att ? 4 : 2;  // weight units per layer: A, C, D, E or D, E
  const int nlu = per_layer * L;

  // this workgroup's row ranges (fixed for all layers)
  int a0, a1, c0, c1, z0, z1, e0, e1, h0, h1;
  split(GW, R, r, a0, a1);
  split(H, R, r, c0, c1);
  split(FS, R, r, z0, z1);
  split(H, R, r, e0, e1);
  split(p.V, nb, b, h0, h1);
  const int lgH = chunk_lg(H, VN), rpbH = kSlots >> lgH;
  const int NHU = p.nhu;

  if (tid == 0) {
    ctl.abort = 0;
    ctl.exbar = 0;
    ctl.pub = 0;
  }

  if (mem) {
    // ================================================================ memory waves
    const int w = wave;
#ifdef QDEC_TRACE
    // memory wave 0's stamps of units 4..15 of the first step, kept in LDS so
    // that no store disturbs the wave's load counting
    constexpr int kMTrace = 72;
    __shared__ u64 mtr[kMTrace];
#define MTRACE(k, s)                                                                              \
  do {                                                                                            \
    if (step == 0 && w == 0 && ml == 0 && (k) >= 4 && (k) < 16) mtr[((k) - 4) * 6 + (s)] = now(); \
  } while (0)
#else
#define MTRACE(k, s) \
  do {               \
  } while (0)
#endif
    Ring rg{ring0 + w * kSlots * kSlotBytes, ring1 + w * kSlots * kSlotBytes, 0, 0, 0,
            sring0 + w * kScaleRegion, sring1 + w * kScaleRegion};
    // the four layer jobs A, C, D, E: slots issued, chunk rows per row (lg),
    // last chunk, and lane q of tab = byte offset of slot q's row from the matrix base
    const Job jobs[4] = {Job{H, 0, H, a1 - a0, 1, a0}, Job{NQ * D, X * QD, QD, c1 - c0, 0, c0},
                         Job{H, 0, H, 2 * (z1 - z0), 2, X * FS + z0}, Job{F, X * FS, FS, e1 - e0, 0, e0}};
    // Short rows of the linear jobs (C, E) are packed 2^pk to a slot. Lane q
    // of tab = byte offset of slot q's (first) row. Int8 weights: lane 4 q + i
    // of stab = byte offset (from the job's scale base) of the i-th 16 bytes
    // of slot q's 64 scale bytes (2^pk row segments of 64 / 2^pk bytes).
    int tab[4], ns[4], lgs[4], nchm1[4], stab[4], pkl[4], nrws[4], rstr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const Job& jb = jobs[t];
      const int lg = chunk_lg(jb.K, VN);
      const int pk = (jb.kind == 0 && lg == 0) ? pack_lg(jb.K, VN) : 0;
      const int nrw = jb.nrows > w ? (jb.nrows - w + kMemWaves - 1) / kMemWaves : 0;
      const int nsl = pk ? (nrw + (1 << pk) - 1) >> pk : nrw << lg;
      lgs[t] = lg;
      ns[t] = __builtin_amdgcn_readfirstlane(nsl);
      nchm1[t] = jb.K / VN - 1;
      pkl[t] = pk;
      nrws[t] = nrw;
      rstr[t] = kMemWaves * jb.ld * ES;
      int ro = 0;
      if (lane < nsl) {
        const int j = w + kMemWaves * (pk ? lane << pk : lane >> lg);
        ro = (jb.phys(j, QD, D, NQ * D, NKV * D, X) * jb.ld + jb.col0) * ES;
      }
      tab[t] = ro;
      int so = 0;
      if (Q8 && lane < 4 * nsl) {
        const int q = lane >> 2, i = lane & 3;
        const int row = min((q << pk) + ((i << pk) >> 2), nrw - 1);
        const int ph = jb.phys(w + kMemWaves * row, QD, D, NQ * D, NKV * D, X);
        so = (ph * (jb.ld / jb.K) + jb.col0 / jb.K) * q8_seg_bytes(jb.K) + ((16 * i) & ((64 >> pk) - 1));
      }
      stab[t] = so;
    }
    const int nrwH = (h1 - h0) > w ? ((h1 - h0) - w + kMemWaves - 1) / kMemWaves : 0;
    const int n_units = nlu + NHU;
    const char* wbase = (const char*)p.wbuf;
    const char* ebase = (const char*)p.embed;
    const char* wsbase = (const char*)p.wscale;
    const char* esbase = (const char*)p.escale;
    const int spH = q8_seg_bytes(H);
    const int rowH = H * ES;
    const int nchH = H / VN - 1;
    int ml = lane;  // made opaque per unit, like the exchange waves' indices

    // issue unit k of a step (weights do not change between steps) into region P
    auto issue = [&](auto par_tag, int k) __attribute__((always_inline)) {
      constexpr int P = decltype(par_tag)::value;
      if (k < nlu) {
        const int l = k / per_layer;
        const int t = k % per_layer + (has_att ? 0 : 2);
        const int tb = t == 0 ? tab[0] : t == 1 ? tab[1] : t == 2 ? tab[2] : tab[3];
        const int n = t == 0 ? ns[0] : t == 1 ? ns[1] : t == 2 ? ns[2] : ns[3];
        const int lg = t == 0 ? lgs[0] : t == 1 ? lgs[1] : t == 2 ? lgs[2] : lgs[3];
        const int cm = t == 0 ? nchm1[0] : t == 1 ? nchm1[1] : t == 2 ? nchm1[2] : nchm1[3];
        const size_t toff = t == 0 ? 0 : t == 1 ? p.off_o : t == 2 ? p.off_gu : p.off_d;
        const char* base = wbase + ((size_t)l * p.layer_elems + toff) * ES;
        const int so = t == 0 ? stab[0] : t == 1 ? stab[1] : t == 2 ? stab[2] : stab[3];
        const size_t stoff = t == 0 ? 0 : t == 1 ? p.soff_o : t == 2 ? p.soff_gu : p.soff_d;
        const Pack pkd{t == 0 ? pkl[0] : t == 1 ? pkl[1] : t == 2 ? pkl[2] : pkl[3],
                       t == 0 ? nrws[0] : t == 1 ? nrws[1] : t == 2 ? nrws[2] : nrws[3],
                       t == 0 ? rstr[0] : t == 1 ? rstr[1] : t == 2 ? rstr[2] : rstr[3]};
        issue_unit<P, Q8>(rg, base, tb, n, lg, cm, ml, wsbase + (size_t)l * p.layer_sbytes + stoff, so, pkd);
      } else {
        const int u = k - nlu;
        const int i0 = u * rpbH;  // first local head row of the unit
        int n = nrwH - i0;
        n = n < 0 ? 0 : (n > rpbH ? rpbH : n);
        const int ro = (h0 + w + kMemWaves * (i0 + (ml >> lgH))) * rowH;
        // int8: one chunk row per head row, so scale lane 4 q + i serves row q
        const int so = Q8 ? (h0 + w + kMemWaves * (i0 + (ml >> 2))) * spH + 16 * (ml & 3) : 0;
        issue_unit<P, Q8>(rg, ebase, ro, __builtin_amdgcn_readfirstlane(n << lgH), lgH, nchH, ml, esbase, so,
                          Pack{0, 0, 0});
      }
    };
    // chunk rows per row, rows per slot and slots of unit k
    auto unit_lg = [&](int k) __attribute__((always_inline)) {
      if (k >= nlu) return lgH;
      const int t = k % per_layer + (has_att ? 0 : 2);
      return t == 0 ? lgs[0] : t == 1 ? lgs[1] : t == 2 ? lgs[2] : lgs[3];
    };
    auto unit_pk = [&](int k) __attribute__((always_inline)) {
      if (k >= nlu) return 0;
      const int t = k % per_layer + (has_att ? 0 : 2);
      return t == 0 ? pkl[0] : t == 1 ? pkl[1] : t == 2 ? pkl[2] : pkl[3];
    };
    auto unit_ns = [&](int k) __attribute__((always_inline)) {
      if (k >= nlu) {
        const int i0 = (k - nlu) * rpbH;
        const int n = nrwH - i0;
        return (n < 0 ? 0 : (n > rpbH ? rpbH : n)) << lgH;
      }
      const int t = k % per_layer + (has_att ? 0 : 2);
      return t == 0 ? ns[0] : t == 1 ? ns[1] : t == 2 ? ns[2] : ns[3];
    };

    if (p.nsteps > 0) issue(std::integral_constant<int, 0>{}, 0);
    if (p.nsteps > 0 && n_units > 1) issue(std::integral_constant<int, 1>{}, 1);
    bar();  // start
    int g = 0;        // units consumed so far (ring parity)
    int pubw = 0;     // publishes to wait for before the next issue
    for (int step = 0; step < p.nsteps; ++step) {
      for (int k = 0; k < n_units; ++k) {
        asm volatile("" : "+v"(ml));
        const bool head = k >= nlu;
        MTRACE(k, 0);
        if (!head || k == nlu) bar();  // input ready
        float* dst = sbuf + (head ? (w * NHU + (k - nlu)) * kSlots : w * kLayerRes);
        const int lg = unit_lg(k), pku = unit_pk(k), nsu = __builtin_amdgcn_readfirstlane(unit_ns(k));
        int kk = k + 2, st = step;
        if (kk >= n_units) {
          kk -= n_units;
          ++st;
        }
        MTRACE(k, 1);
        if (g & 1) {
          ring_wait<1>(rg);
          MTRACE(k, 2);
          consume_unit<1, WT>(rg, lg, pku, nsu, xin, dst, ml);
          MTRACE(k, 3);
          if (!head) {
            bar();  // partials ready
            pubw += kExWaves;
            wait_published(pubw, &ctl, p.err);
          }
          MTRACE(k, 4);
          if (st < p.nsteps) issue(std::integral_constant<int, 1>{}, kk);
        } else {
          ring_wait<0>(rg);
          MTRACE(k, 2);
          consume_unit<0, WT>(rg, lg, pku, nsu, xin, dst, ml);
          MTRACE(k, 3);
          if (!head) {
            bar();  // partials ready
            pubw += kExWaves;
            wait_published(pubw, &ctl, p.err);
          }
          MTRACE(k, 4);
          if (st < p.nsteps) issue(std::integral_constant<int, 0>{}, kk);
        }
        MTRACE(k, 5);
        if (head && k == n_units - 1) bar();  // LM-head partials ready
        ++g;
      }
    }
#ifdef QDEC_TRACE
    if (w == 0 && ml == 0)
      for (int i = 0; i < kMTrace; ++i) g_trace[blockIdx.x * kTraceN + 320 + i] = mtr[i];
#endif
    return;
  }

  // ================================================================== exchange waves
  // Raised issue priority: on the SIMDs they share with the memory waves, the
  // exchange waves' instructions (the latency-bound chain) are issued first.
  __builtin_amdgcn_s_setprio(2);
  // Per-thread indices and the parameter block are made opaque at the top of
  // every layer: keeps address arithmetic from being hoisted out of the loops
  // and pinned in registers for the whole launch.
  int et = tid - kExBase;
  int ln = lane;
  const int ew = wave - kMemWaves;
  int exgen = 0;
  // the kernel's only argument sits at the start of the kernel-argument segment;
  // reading it through a constant-address-space pointer keeps the loads scalar
  typedef const __attribute__((address_space(4))) DecParams* ParamPtr;
  ParamPtr pp = (ParamPtr)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int half = D / 2;
  // gains (loaded one use ahead): in-norm (or final) and post-norm of this
  // thread's residual elements, and Q/K-norm gains of this wave's head vectors
  float gi[NE], gp[NE], gq[2][2];
  auto load_in = [&](int l) __attribute__((always_inline)) {
    const float* g = l < L ? pp->nbuf + (size_t)l * pp->norm_elems : pp->final_norm;
#pragma unroll
    for (int k = 0; k < NE; ++k) gi[k] = g[min(et + k * kEx, H - 1)];
  };
  auto load_post = [&](int l) __attribute__((always_inline)) {
    const float* g = pp->nbuf + (size_t)l * pp->norm_elems + H;
#pragma unroll
    for (int k = 0; k < NE; ++k) gp[k] = g[min(et + k * kEx, H - 1)];
  };
  // this wave's head vectors hv = ew, ew + 4 of the (G + 2) in Lq: q heads, k, v
  auto load_qk = [&](int l) __attribute__((always_inline)) {
    const float* g = pp->nbuf + (size_t)l * pp->norm_elems + 2 * H;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int hv = ew + kExWaves * i;
      const float* gg = hv < G ? g : g + D;  // q_norm, else k_norm
      const int hl = ln < half ? ln : 0;
      gq[i][0] = gg[hl];
      gq[i][1] = gg[hl + half];
    }
  };
  float x[NE];  // residual stream: elements et + k * kEx
  const float inv_h = 1.f / (float)H;
  // GEMV input x * g and this wave's sum of squares of x
  auto norm_input = [&](const float (&g)[NE]) __attribute__((always_inline)) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      const int e = et + k * kEx;
      if (e < H) {
        ss = fmaf(x[k], x[k], ss);
        xin[e] = x[k] * g[k];
      }
    }
    ss = wave_sum(ss);
    if (ln == 0) ctl.red[ew] = ss;
  };
  auto norm_scale = [&]() __attribute__((always_inline)) {
    const float ss = 0.f + ctl.red[0] + ctl.red[1] + ctl.red[2] + ctl.red[3];
    return 1.f / sqrtf(ss * inv_h + pp->eps);
  };
  // zero the GEMV input from n to the end of its last 64-lane chunk row
  auto pad = [&](int n) __attribute__((always_inline)) {
    const int end = (kWave * VN) << chunk_lg(n, VN);
    for (int i = n + et; i < end; i += kEx) xin[i] = 0.f;
  };
  // combined dot of local row j of a layer unit with 2^lg chunk rows per row
  // (packed units have lg 0: row i's total is entry i)
  auto row_val = [&](int j, int lg) __attribute__((always_inline)) {
    const int w = j & (kMemWaves - 1), i = j >> 2;
    const float* s = sbuf + w * kLayerRes + (i << lg);
    float v = s[0];
    for (int jj = 1; jj < (1 << lg); ++jj) v += s[jj];
    return v;
  };

  load_in(0);
  load_post(0);
  load_qk(0);
  {
    const int np = (pp->pos0 + pp->nsteps + kPage - 1) / kPage;  // <= kPtabLds (checked by the host)
    for (int i = et; i < np; i += kEx) ptab[i] = (u64)pp->page_table[i];
  }
  int token = pp->token_dev ? pp->token_dev[0] : pp->token;
  token = token < 0 ? 0 : (token >= pp->V ? pp->V - 1 : token);
  bar();  // start

  for (int step = 0; step < pp->nsteps; ++step) {
    const int pos = pp->pos0 + step;
    const int n_hist = pos;  // cached positions 0 .. pos-1
    float rc = 1.f, rs = 0.f;
    if (ln < half) {
      rc = pp->rope_cos[(size_t)pos * half + ln];
      rs = pp->rope_sin[(size_t)pos * half + ln];
    }
    if constexpr (Q8) {
      const int8_t* ec = (const int8_t*)pp->embed + (size_t)token * H;
      const unsigned short* es = (const unsigned short*)((const char*)pp->escale + (size_t)token * q8_seg_bytes(H));
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int e = min(et + k * kEx, H - 1);
        x[k] = (float)ec[e] * half_bits(es[e / kQ8Block]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NE; ++k) x[k] = wload((const WT*)pp->embed, (size_t)token * H + min(et + k * kEx, H - 1));
    }
    TRACE(step, 0);
    // attention mode for this step
    const bool whole = n_hist <= pp->whole_max;
    int nsplit = 1, per = n_hist;
    if (!whole) {
      // splits of whole pages; nsplit recounted so that none is empty
      nsplit = min(pp->nsplit_max, (n_hist + pp->whole_max - 1) / pp->whole_max);
      per = ((n_hist + nsplit - 1) / nsplit + kPage - 1) / kPage * kPage;
      nsplit = (n_hist + per - 1) / per;
    }
    const bool att_rank = whole || r < nsplit;
    int u0 = 0, n_cached = n_hist;
    if (!whole) {
      u0 = min(n_hist, r * per);
      n_cached = min(n_hist, u0 + per) - u0;
    }
    // cached K/V of a layer's first two attention iterations do not depend on
    // the token: they are loaded one phase ahead, under an exchange wait
    Attn<D, G> at;
    if (has_att && att_rank) at.prefetch(p, ptab, 0, X, u0, n_cached, ew, ln);

    for (int l = 0; l <= L; ++l) {
      QDEC_OPAQUE();
      const int gl = step * L + l;
      const int par = gl & 1, ppar = par ^ 1;
      const unsigned tg = pp->tag0 + (unsigned)((step * (L + 1) + l) * kTagSlots);
      const unsigned tgp = tg - kTagSlots;  // layer l-1 of this step
      if (l > 0) {
        const u64* Lx_prev = pp->ll + pp->o_x + (size_t)ppar * kGroups * H;
        u64* Lxs_prev = pp->ll + pp->o_xs + ((size_t)ppar * kGroups + X) * H;
        reduce2<NE>(Lx_prev, kGroups, H, e0, e1, tgp + PH_X, Lxs_prev, tgp + PH_XS, x, et, &ctl, pp->err, pp->local);
      }
      TRACE(step, 1 + l * 10 + 0);
#ifdef QDEC_TRACE
      // shader-clock counter beside the 100 MHz counter (clock-rate check)
      if (step == 0 && tid == kExBase && (l == 2 || l == 12)) g_xtr[l == 2 ? 504 : 505] = __builtin_amdgcn_s_memtime();
#endif
      if (l == L) break;
      u64* Lq = pp->ll + pp->o_q + ((size_t)par * NKV + X) * GW;
      u64* La = pp->ll + pp->o_att + ((size_t)par * NKV + X) * R * G * (D + 2);
      u64* Lo = pp->ll + pp->o_o + (size_t)par * NKV * H;
      u64* Lz = pp->ll + pp->o_z + ((size_t)par * kGroups + X) * FS;
      u64* Lx = pp->ll + pp->o_x + (size_t)par * kGroups * H;

      if (has_att) {
        // ---------------- A
        norm_input(gi);
        pad(H);
        if (l < 8) TRACE(step, 400 + l * 4 + 0);
        bar();  // input ready
        bar();  // partials ready
        TRACE(step, 1 + l * 10 + 1);
        {
          const float inv = norm_scale();
          const int lg = chunk_lg(H, VN);
          for (int j = et; j < a1 - a0; j += kEx) put_l(Lq + a0 + j, inv * row_val(j, lg), tg + PH_Q, pp->local);
        }
        published(ln, &ctl);
        TRACEB(step, l, 0);
        // ---------------- B: this wave's head vectors from the group's Q/K/V rows
        QDEC_OPAQUE();
        float va[2], vb[2];
        {
          const u64 t0 = now();
          u64 w[2][2];
          const int hl = ln < half ? ln : 0;
          const int hv0 = min(ew, G + 1), hv1 = min(ew + kExWaves, G + 1);
          while (true) {
            get_l4(Lq + hv0 * D + hl, Lq + hv0 * D + hl + half, Lq + hv1 * D + hl, Lq + hv1 * D + hl + half,
                   w[0][0], w[0][1], w[1][0], w[1][1], pp->local);
            const bool done = tagged(w[0][0], tg + PH_Q) && tagged(w[0][1], tg + PH_Q) &&
                              tagged(w[1][0], tg + PH_Q) && tagged(w[1][1], tg + PH_Q);
            if (done || give_up(t0, &ctl, pp->err)) break;
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            va[i] = val(w[i][0]);
            vb[i] = val(w[i][1]);
          }
        }
        TRACE(step, 1 + l * 10 + 2);
        // per-head RMSNorm + RoPE (q heads, k); v copied; rank 0 appends K and V at pos
        {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int hv = ew + kExWaves * i;
            if (hv > G + 1) continue;  // wave-uniform
            float a = ln < half ? va[i] : 0.f, c = ln < half ? vb[i] : 0.f;
            if (hv <= G) {
              const float ssq = wave_sum(a * a + c * c);
              const float inv = 1.f / sqrtf(ssq / (float)D + pp->eps);
              a = a * inv * gq[i][0];
              c = c * inv * gq[i][1];
              const float ra = a * rc - c * rs, rb = c * rc + a * rs;
              a = ra;
              c = rb;
            }
            if (ln < half) {
              if (hv < G) {
                q_l[hv * QS + Attn<D, G>::padi(ln)] = a * pp->scale;
                q_l[hv * QS + Attn<D, G>::padi(ln + half)] = c * pp->scale;
              } else if (hv == G) {
                k_l[Attn<D, G>::padi(ln)] = a;
                k_l[Attn<D, G>::padi(ln + half)] = c;
              } else {
                v_l[ln] = a;
                v_l[ln + half] = c;
              }
            }
          }
        }
        TRACEB(step, l, 2);
        ex_sync(exgen, ln, &ctl, pp->err);
        TRACEB(step, l, 3);
        if (att_rank)
          at.partial(p, ptab, l, X, u0, n_cached, whole || r == nsplit - 1, q_l, k_l, v_l,
                     pw + ew * G * Attn<D, G>::KPW, wm, wl, wo, ew, ln, step, tid);
        TRACEB(step, l, 4);
        ex_sync(exgen, ln, &ctl, pp->err);
        TRACEB(step, l, 5);
        TRACE(step, 1 + l * 10 + 3);
        // ---------------- C input: o of the G heads, merged over waves (and splits)
        QDEC_OPAQUE();
        if (whole) {
          for (int idx = et; idx < QD; idx += kEx) {
            const int h = idx / D, d = idx % D;
            float M = -INFINITY;
#pragma unroll
            for (int w2 = 0; w2 < kExWaves; ++w2) M = fmaxf(M, wm[w2 * G + h]);
            float lt = 0.f, o = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < kExWaves; ++w2) {
              const float mw = wm[w2 * G + h];
              const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
              lt = fmaf(f, wl[w2 * G + h], lt);
              o = fmaf(f, wo[(w2 * G + h) * D + d], o);
            }
            xin[idx] = o / lt;
          }
        } else {
          if (r < nsplit) {
            for (int idx = et; idx < G * (D + 2); idx += kEx) {
              const int h = idx / (D + 2), e = idx % (D + 2);
              float M = -INFINITY;
#pragma unroll
              for (int w2 = 0; w2 < kExWaves; ++w2) M = fmaxf(M, wm[w2 * G + h]);
              float v = M;
              if (e > 0) {
                v = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < kExWaves; ++w2) {
                  const float mw = wm[w2 * G + h];
                  const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                  v = fmaf(f, e == 1 ? wl[w2 * G + h] : wo[(w2 * G + h) * D + (e - 2)], v);
                }
              }
              put_l(La + (size_t)r * G * (D + 2) + idx, v, tg + PH_ATT, pp->local);
            }
          }
          // Merge in two light stages instead of every rank reading every
          // split's partials: rank r merges outputs [j0, j0 + per) of the
          // G * D, reading only their (m, l, o) words of each split, and
          // publishes them; every rank then collects the merged vector.
          const int mper = (QD + R - 1) / R, j0 = min(QD, r * mper), jn = min(mper, QD - j0);
          float* m2 = stage;                  // [split][mper]
          float* l2 = m2 + nsplit * mper;
          float* o2 = l2 + nsplit * mper;
          for (int t = et; t < nsplit * mper; t += kEx) {
            const int sp = t / mper, jj = t % mper, j = min(j0 + jj, QD - 1);
            const u64* base = La + (size_t)sp * G * (D + 2) + (j / D) * (D + 2);
            const u64 t0 = now();
            u64 wv[4];
            while (true) {
              get_l4(base, base + 1, base + 2 + j % D, base + 2 + j % D, wv[0], wv[1], wv[2], wv[3], pp->local);
              if ((tagged(wv[0], tg + PH_ATT) && tagged(wv[1], tg + PH_ATT) && tagged(wv[2], tg + PH_ATT)) ||
                  give_up(t0, &ctl, pp->err))
                break;
            }
            m2[t] = val(wv[0]);
            l2[t] = val(wv[1]);
            o2[t] = val(wv[2]);
          }
          ex_sync(exgen, ln, &ctl, pp->err);
          u64* Lm = pp->ll + pp->o_att2 + ((size_t)par * NKV + X) * QD;
          for (int jj = et; jj < jn; jj += kEx) {
            float M = -INFINITY;
            for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, m2[sp * mper + jj]);
            float o = 0.f, lt = 0.f;
            for (int sp = 0; sp < nsplit; ++sp) {
              const float ms = m2[sp * mper + jj];
              const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
              o = fmaf(f, o2[sp * mper + jj], o);
              lt = fmaf(f, l2[sp * mper + jj], lt);
            }
            put_l(Lm + j0 + jj, o / lt, tg + PH_ATT, pp->local);
          }
          gather_local(Lm, QD, tg + PH_ATT, xin, et, &ctl, pp->err, pp->local);
        }
        pad(QD);
        // rank 0 appends this token's K and V at pos (device scope: other CUs
        // of the group read them in later steps). Stores count against the
        // same in-order counter as loads, so they are issued only after the
        // attention; they complete before this workgroup publishes again.
        if (r == 0) {
          gfloat* page = page_of(ptab, pos);
          Dims dd{L, 0, 0, NKV, D, 0, 0, 0.f};
          for (int i = et; i < 2 * D; i += kEx) {
            const int sel = i / D, d = i % D;
            __hip_atomic_store(page + page_offset(dd, l, sel, X, pos % kPage) + d,
                               sel ? v_l[d] : k_l[Attn<D, G>::padi(d)],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        // next layer's gains: a wave's loads retire in order, so these are
        // issued only now, ahead of the O-partial wait that hides them
        load_in(l + 1);
        if (l + 1 < L) load_qk(l + 1);
        TRACE(step, 1 + l * 10 + 4);
        bar();  // input ready
        bar();  // partials ready
        {
          const int lg = chunk_lg(QD, VN);
          for (int j = et; j < c1 - c0; j += kEx) put(Lo + (size_t)X * H + c0 + j, row_val(j, lg), tg + PH_O);
        }
        published(ln, &ctl);
      } else {
        load_in(l + 1);
      }

      // ---------------- D
      QDEC_OPAQUE();
      TRACE(step, 1 + l * 10 + 5);
      // rank 0's K/V append stores are complete before anything else of this
      // workgroup is published (a later step reads them from other CUs)
      if (has_att && r == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
      {
        u64* Los = pp->ll + pp->o_os + ((size_t)par * kGroups + X) * H;
        reduce2<NE>(Lo, NKV, H, c0, c1, tg + PH_O, Los, tg + PH_OS, x, et, &ctl, pp->err, pp->local);
      }
      TRACE(step, 1 + l * 10 + 6);
      norm_input(gp);
      pad(H);
      if (l + 1 < L) load_post(l + 1);
      if (l < 8) TRACE(step, 400 + l * 4 + 1);
      bar();  // input ready
      bar();  // partials ready
      if (l < 8) TRACE(step, 400 + l * 4 + 2);
      {
        const float inv = norm_scale();
        const int lg = chunk_lg(H, VN);
        for (int i = et; i < z1 - z0; i += kEx) {
          const float gt = inv * row_val(2 * i, lg), up = inv * row_val(2 * i + 1, lg);
          put_l(Lz + z0 + i, gt / (1.f + expf(-gt)) * up, tg + PH_Z, pp->local);
        }
      }
      published(ln, &ctl);
      TRACE(step, 1 + l * 10 + 7);

      // ---------------- E
      QDEC_OPAQUE();
      gather_local(Lz, FS, tg + PH_Z, xin, et, &ctl, pp->err, pp->local);
      pad(FS);
      TRACE(step, 1 + l * 10 + 8);
      bar();  // input ready
      // cached K/V of the next layer's first attention block do not depend on
      // the token: their loads are issued while the memory waves run the down
      // dot, so issuing them costs the exchange waves no time on the chain
      if (has_att && att_rank && l + 1 < L) at.prefetch(p, ptab, l + 1, X, u0, n_cached, ew, ln);
      bar();  // partials ready
      if (l < 8) TRACE(step, 400 + l * 4 + 3);
      {
        const int lg = chunk_lg(FS, VN);
        for (int j = et; j < e1 - e0; j += kEx) put(Lx + (size_t)X * H + e0 + j, row_val(j, lg), tg + PH_X);
      }
      published(ln, &ctl);
      TRACE(step, 1 + l * 10 + 9);
    }

    // ---------------- final RMSNorm + tied LM head + greedy argmax
    QDEC_OPAQUE();
    norm_input(gi);
    pad(H);
    load_in(0);
    load_post(0);
    load_qk(0);
    bar();  // input ready
    bar();  // LM-head partials ready
    TRACE(step, 300);
    u64 best = 0ull;
    {
      const float inv = norm_scale();
      float* lg_out = pp->logits ? pp->logits + (size_t)step * pp->V + h0 : nullptr;
      for (int j = et; j < h1 - h0; j += kEx) {
        const int w = j & (kMemWaves - 1), i = j >> 2;
        const int u = i / rpbH, ii = i - u * rpbH;
        const float* s = sbuf + (w * NHU + u) * kSlots + (ii << lgH);
        float v = s[0];
        for (int jj = 1; jj < (1 << lgH); ++jj) v += s[jj];
        v *= inv;
        if (lg_out) lg_out[j] = v;
        best = umax64(best, argmax_key(v, h0 + j));
      }
    }
    best = wave_max64(best);
    if (ln == 0) ctl.best[0][ew] = best;
    ex_sync(exgen, ln, &ctl, pp->err);
    const int kpar = step & 1;
    u64* Lk = pp->ll + pp->o_key + (size_t)kpar * 2 * nb;
    const unsigned ktag = pp->tag0 + (unsigned)((step * (L + 1) + L) * kTagSlots) + PH_KEY;
    if (et == 0) {
      u64 b2 = ctl.best[0][0];
      for (int i = 1; i < kExWaves; ++i) b2 = umax64(b2, ctl.best[0][i]);
      put(Lk + 2 * b, __uint_as_float((unsigned)(b2 >> 32)), ktag);
      put(Lk + 2 * b + 1, __uint_as_float((unsigned)b2), ktag);
    }
    TRACE(step, 301);
    const bool need = (step + 1 < pp->nsteps) || b == 0;
    if (need) {
      // thread et < nb reads workgroup et's key
      u64 kb;
      {
        const int i = min(et, nb - 1);
        const u64 t0 = now();
        u64 w0, w1;
        while (true) {
          w0 = get(Lk + 2 * i);
          w1 = get(Lk + 2 * i + 1);
          if ((tagged(w0, ktag) && tagged(w1, ktag)) || give_up(t0, &ctl, pp->err)) break;
        }
        kb = ((u64)(unsigned)w0 << 32) | (u64)(unsigned)w1;
      }
      kb = wave_max64(kb);
      if (ln == 0) ctl.best[1][ew] = kb;
      ex_sync(exgen, ln, &ctl, pp->err);
      u64 b3 = ctl.best[1][0];
      for (int i = 1; i < kExWaves; ++i) b3 = umax64(b3, ctl.best[1][i]);
      token = (int)(0xFFFFFFFFu - (uint32_t)(b3 & 0xFFFFFFFFull));
      token = token < 0 ? 0 : (token >= pp->V ? pp->V - 1 : token);
      if (b == 0 && et == 0) pp->tokens_out[step] = token;
      TRACE(step, 302);
    }
  }
#ifdef QDEC_TRACE
  if (tid == kExBase)
    for (int i = 0; i < 320; ++i) g_trace[blockIdx.x * kTraceN + i] = g_xtr[i];
  if (tid == kExBase)
    for (int i = 392; i < kTraceN; ++i) g_trace[blockIdx.x * kTraceN + i] = g_xtr[i];
#endif
}

// Dynamic LDS layout (floats): stage | att | sbuf | ptab (u64)
struct Layout {
  int stage, att, sbuf, ptab, total, nhu;
};
// inputs per 16-byte chunk for a weight kind (QDEC_F32, QDEC_BF16, QDEC_Q8_0)
int chunk_elems(int wt) { return wt == QDEC_BF16 ? 8 : wt == QDEC_Q8_0 ? 16 : 4; }

Layout layout(int wt, const Dims& d, int nsplit_max, int nb) {
  const int G = d.NQ / d.NKV;
  const int VN = chunk_elems(wt);
  const int per = (G * d.D + nb / kGroups - 1) / (nb / kGroups);  // merged outputs per rank
  const int stage = std::max(8, 3 * nsplit_max * per);            // split merge: (m, l, o) per split
  const int qs = d.D + 16;  // padded q/k row (4 floats after each quarter)
  const int att = (G + 1) * qs + d.D + 2 * kExWaves * G + kExWaves * G * d.D + kExWaves * G * (kWave / 4);
  const int hrows = (d.V + nb - 1) / nb;
  const int rows_w = (hrows + kMemWaves - 1) / kMemWaves;
  const int rpb = kSlots >> chunk_lg(d.H, VN);
  Layout o;
  o.nhu = std::max(1, (rows_w + rpb - 1) / rpb);
  o.stage = 0;
  o.att = o.stage + ((stage + 3) & ~3);
  o.sbuf = o.att + ((att + 3) & ~3);
  o.ptab = o.sbuf + ((std::max(kMemWaves * o.nhu * kSlots, kMemWaves * kLayerRes) + 3) & ~3);
  o.total = o.ptab + 2 * kPtabLds;
  return o;
}

const void* kernel_for(int wt, const Dims& d) {
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
  if (wt == QDEC_BF16) {
    QDEC_DEC_ALL(uint16_t)
  } else if (wt == QDEC_Q8_0) {
    QDEC_DEC_ALL(int8_t)
  } else {
    QDEC_DEC_ALL(float)
  }
#undef QDEC_DEC_ALL
#undef QDEC_DEC_CASE
  return nullptr;
}

}  // namespace

size_t dec_lds_bytes(int wt, const Dims& d, int nblocks, int nsplit_max) {
  return (size_t)layout(wt, d, nsplit_max, nblocks).total * sizeof(float);
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
  off->os = o; o += 2 * (size_t)kGroups * d.H;
  off->xs = o; o += 2 * (size_t)kGroups * d.H;
  off->att2 = o; o += 2 * (size_t)d.NKV * G * d.D;
  return o;
}

unsigned dec_tags_per_step(const Dims& d) { return (unsigned)((d.L + 1) * kTagSlots); }

// Every GEMV input fits the LDS input vector and every layer phase of a
// workgroup fits one ring region per memory wave: (rows per wave) * (chunk
// rows per row) <= kSlots; at most one argmax key per exchange thread. Int8
// weights also need every dot's input length to be whole scale blocks.
bool dec_fits(int wt, const Dims& d, int nblocks) {
  if (nblocks < kGroups || nblocks % kGroups || nblocks > kMaxBlocks) return false;
  const int R = nblocks / kGroups;
  const int VN = chunk_elems(wt);
  const int G = d.NQ / d.NKV;
  const int FS = d.F / kGroups;
  // packable: consecutive rows a fixed stride apart (the linear jobs C, E)
  auto fits = [&](int rows_per_block, int K, bool packable) {
    if (K > kMaxK || K % VN) return false;
    if (wt == QDEC_Q8_0 && K % kQ8Block) return false;
    const int rows_w = (rows_per_block + kMemWaves - 1) / kMemWaves;
    const int lg = chunk_lg(K, VN);
    const int pk = (packable && lg == 0) ? pack_lg(K, VN) : 0;
    return (pk ? (rows_w + (1 << pk) - 1) >> pk : rows_w << lg) <= kSlots;
  };
  auto per = [&](int n) { return (n + R - 1) / R; };
  return fits(per((G + 2) * d.D), d.H, false) && fits(per(d.H), G * d.D, true) && fits(2 * per(FS), d.H, false) &&
         fits(per(d.H), FS, true) && fits(1, d.H, false);
}

int dec_split_limit(const Dims& d, int nblocks) {
  (void)d;
  // every rank of a group may take a split (the partial words hold R splits)
  return std::max(1, nblocks / kGroups);
}

hipError_t dec_prepare(int wt, const Dims& d, size_t lds, int* blocks_per_cu) {
  const void* fn = kernel_for(wt, d);
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
  p.wscale = a.wscale;
  p.layer_sbytes = a.layer_sbytes;
  p.soff_o = a.soff_o;
  p.soff_gu = a.soff_gu;
  p.soff_d = a.soff_d;
  p.escale = a.escale;
  p.final_norm = a.final_norm;
  p.rope_cos = a.rope_cos;
  p.rope_sin = a.rope_sin;
  p.page_table = a.page_table;
  p.L = d.L; p.H = d.H; p.NQ = d.NQ; p.NKV = d.NKV; p.F = d.F; p.V = d.V;
  p.eps = d.eps;
  // scores in base 2: q carries log2(e) / sqrt(D), the softmax uses exp2
  p.scale = 1.4426950408889634f / sqrtf((float)d.D);
  p.pos0 = a.pos;
  p.nsteps = a.nsteps;
  p.token = a.token;
  p.token_dev = a.token_dev;
  p.logits = a.logits;
  p.tokens_out = a.tokens_out;
  p.ll = a.ll;
  p.o_q = a.off.q; p.o_att = a.off.att; p.o_o = a.off.o; p.o_z = a.off.z; p.o_x = a.off.x; p.o_key = a.off.key;
  p.o_os = a.off.os; p.o_xs = a.off.xs; p.o_att2 = a.off.att2;
  p.tag0 = a.tag0;
  p.err = a.err;
  p.local = a.local ? 1 : 0;
  p.R = a.nblocks / kGroups;
  p.nsplit_max = a.nsplit_max;
  p.whole_max = a.whole_max;
  const Layout lay = layout(a.wt, d, a.nsplit_max, a.nblocks);
  p.nhu = lay.nhu;
  p.lds_stage = lay.stage; p.lds_att = lay.att; p.lds_sbuf = lay.sbuf; p.lds_ptab = lay.ptab;
  const void* fn = kernel_for(a.wt, d);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {&p};
  // A plain launch: one workgroup per CU (the LDS footprint allows no more),
  // as many workgroups as CUs, so on a device this process has to itself all
  // of them are resident at once. Residency is not assumed for safety: every
  // cross-CU wait has a time limit, so a workgroup that could not start would
  // make the launch report QDEC_E_DEVICE rather than hang. (A cooperative
  // launch costs about 17 us more per call.)
  return hipLaunchKernel(fn, dim3(a.nblocks), dim3(kThreads), args, (unsigned)a.lds_bytes, st);
}

#ifdef QDEC_TRACE
extern "C" int qdec_debug_trace(unsigned long long* host, int n) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_trace), sizeof(unsigned long long) * (size_t)n, 0,
                                  hipMemcpyDeviceToHost);
}
#endif

// Placement probe: thread 0 of each workgroup records the id of the XCD it
// runs on (hardware register XCC_ID, low 4 bits). Launched with the decode
// kernel's grid, block and LDS size, so the dispatcher places it the same way.
__global__ __launch_bounds__(kThreads) void xcc_probe_kernel(int* out) {
  extern __shared__ float probe_lds[];
  if (threadIdx.x == 0) {
    probe_lds[0] = 0.f;
    out[blockIdx.x] = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 0xF);
  }
}

hipError_t launch_xcc_probe(int wt, const Dims& d, int* out_dev, int nblocks, size_t lds_bytes, hipStream_t st) {
  // the probe asks for the decode kernel's whole LDS (static + dynamic), so
  // one workgroup fits per CU as in a decode launch
  const void* fn = kernel_for(wt, d);
  if (!fn) return hipErrorInvalidValue;
  hipFuncAttributes attr{};
  hipError_t e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  const size_t total = attr.sharedSizeBytes + lds_bytes;
  e = hipFuncSetAttribute((const void*)xcc_probe_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)total);
  if (e != hipSuccess) return e;
  xcc_probe_kernel<<<nblocks, kThreads, total, st>>>(out_dev);
  return hipGetLastError();
}

// Fill kernel for the exchange words (used when tags are about to wrap).
__global__ void clear_words_kernel(u64* w, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) w[i] = 0ull;
}

hipError_t launch_clear_words(unsigned long long* w, size_t n, hipStream_t st) {
  clear_words_kernel<<<256, 256, 0, st>>>(w, n);
  return hipGetLastError();
}

}  // namespace qdec
