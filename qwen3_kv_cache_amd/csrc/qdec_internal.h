// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/qdec.h"

namespace qdec {

constexpr int kPage = QDEC_PAGE;   // positions per KV page
constexpr int kGuGroup = 8;        // gate/up rows interleaved in groups of 8 in the packed weight
constexpr int kAttnChunk = 128;    // positions per split in batched decode attention
static_assert(kAttnChunk % kPage == 0, "a split covers whole pages");
constexpr int kMaxBatch = 16;
constexpr int kDecMaxPos = QDEC_DECODE_MAX_POS;  // decode positions (KV page pointers held in LDS)

// Model dimensions as the kernels see them.
struct Dims {
  int L, H, NQ, NKV, D, F, V;
  float eps;
  int qkv() const { return (NQ + 2 * NKV) * D; }
};

// Packed per-layer weights (device). wqkv = [wq; wk; wv] rows; wgu holds
// gate and up rows interleaved in groups of kGuGroup: packed rows
// [16g, 16g+8) are gate rows [8g, 8g+8), packed rows [16g+8, 16g+16) the
// matching up rows.
struct LayerW {
  const void* wqkv;
  const void* wo;
  const void* wgu;
  const void* wd;
  const float* in_norm;
  const float* post_norm;
  const float* q_norm;
  const float* k_norm;
};

// KV page layout (fp32): page[layer][0=K,1=V][kv_head][slot][head_dim].
__host__ __device__ inline size_t page_floats(const Dims& d) {
  return (size_t)d.L * 2 * d.NKV * kPage * d.D;
}
__host__ __device__ inline size_t page_offset(const Dims& d, int layer, int kv, int head, int slot) {
  return ((((size_t)layer * 2 + kv) * d.NKV + head) * kPage + slot) * d.D;
}

// Rows of a batched decode step, passed by value as a kernel argument: row r
// is one state fed token tok[r] at position pos[r], its KV page table at
// pt[r] (device).
struct BatchRows {
  int n;
  int tok[kMaxBatch];
  int pos[kMaxBatch];
  const int64_t* pt[kMaxBatch];
};

// ---- launchers (qdec_kernels.hip); all enqueue on `st`, return hipError_t
// The embed launchers also write each row's sum of squares to ssq[row] when
// ssq is set (the first layer's RMSNorm partials, one per row).
hipError_t launch_embed_rows(const Dims& d, bool bf16, const void* E, const BatchRows& rows, float* X, float* ssq,
                             hipStream_t st);
hipError_t launch_embed_prefill(const Dims& d, bool bf16, const void* E, const int32_t* ids, int T,
                                const float* audio, int a0, int La, float* X, float* ssq, hipStream_t st);

// EPI_SWIGLU_SPLIT (tiled GEMM only): the SwiGLU output written as bf16 hi
// and lo, the next GEMM's operand, instead of fp32
// EPI_RELU (bf16 GEMMs): C = max(v + bias, 0)
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_HEAD = 3, EPI_SWIGLU_SPLIT = 4, EPI_RELU = 5 };

// Arguments of the fused small-M GEMM (gemm_rows_kernel): up to 64 fp32
// activation rows against bf16 weights, optional RMSNorm prologue, split-K
// reduced in a fixed order, epilogue per Epi.
struct RowsGemm {
  const float* A;               // activations [M, lda] (first K columns used)
  int lda;
  const float* ssq;             // NORM: per-row sum-of-squares partials [nss][M]
  int nss;
  const float* gain;            // NORM: gain [K]
  float eps;
  const void* W;                // [N, K], bf16 (fp32 when wf32)
  int wf32;
  int M, K, N;
  int KC;                       // set by the launcher
  unsigned long long* P;        // split-K partial words (rows_partial_floats of them)
  unsigned* cnt;                // arrival counters, zero between launches (rows_counters)
  unsigned tag;                 // nonzero, differs from every tag still held in P
  int* err;                     // set to 1 if a partial never became visible (host-mapped)
  float* C;                     // output; SWIGLU: [M, N/2]; HEAD: logits or null
  int ldc;
  float* ssq_out;               // RESID: [N / rows_tile_cols(N)][M]
  unsigned long long* keys;     // HEAD: argmax key per row
};
bool rows_fits(int M, int K, int N);
int rows_tile_cols(int N);
size_t rows_partial_floats(int M, int K, int N);
int rows_counters(int M, int K, int N);
hipError_t launch_gemm_rows(Epi epi, bool norm, const RowsGemm& g, hipStream_t st);
hipError_t launch_lm_head(const Dims& d, bool bf16, const void* E, const float* x, const float* gain,
                          float* logits, unsigned long long* key, hipStream_t st);
// Argmax keys of a row are spread over kKeySlots words (key[row * kKeySlots
// + slot], the slot picked by the producing block) so that thousands of
// blocks do not all take their atomic max on one word; argmax_final reduces
// the slots.
constexpr int kKeySlots = 16;
hipError_t launch_argmax_final(const unsigned long long* key, int n, int32_t* out, hipStream_t st);
hipError_t launch_reset_keys(unsigned long long* key, int n, hipStream_t st);
// key[r] = max(key[r], argmax key of logits row r), r < n
hipError_t launch_argmax_rows(const float* logits, int n, int V, unsigned long long* key, hipStream_t st);

hipError_t launch_qk_rope_append(const Dims& d, float* qkv, int T, int pos0, const float* q_norm,
                                 const float* k_norm, const float* rope_cos, const float* rope_sin,
                                 const int64_t* page_table, int layer, hipStream_t st);
// Short prompts (T <= kSmallT): per-head Q/K-RMSNorm, RoPE, the K/V append
// of positions [0, T) and causal attention in one launch; out is fp32
// [T][NQ D]. qkv is only read.
constexpr int kSmallT = 64;
bool attn_small_fits(const Dims& d, int T);
hipError_t launch_attn_small(const Dims& d, const float* qkv, int T, const float* q_norm, const float* k_norm,
                             const float* rope_cos, const float* rope_sin, const int64_t* page_table, int layer,
                             float* out, hipStream_t st);
// Batched decode attention for one layer (QK-norm, RoPE and K/V append of
// the rows' current positions included). The launcher fills L, NKV, ld, eps
// and qscale.
struct AttnRows {
  BatchRows rows;
  float* qkv;                   // [n, ld] raw Q | K | V rows of the QKV GEMM
  int ld, L, NKV, layer;
  const float* q_norm;
  const float* k_norm;
  const float* rcos;
  const float* rsin;
  float eps, qscale;
  float* out;                   // [n, NQ * D]
  unsigned long long* part;     // n * NKV * nsplit * GROUP * (D + 2) words
  unsigned* cnt;                // n * NKV counters, zero between launches
  unsigned tag;                 // as RowsGemm::tag
  int* err;
};
// nsplit * kAttnChunk must cover the longest row (pos + 1)
hipError_t launch_attn_rows(const Dims& d, const AttnRows& a, int nsplit, hipStream_t st);
// Causal prefill attention over QKV rows [T, qkv()]. For head_dim 128 with
// GQA 1 or 2 (attn_prefill_uses_split) K and V are first converted into
// kv[0..3] = K hi, K lo ([NKV][T][128] bf16 each) and V^T hi, lo
// ([NKV][128][kv_split_pad(T)] bf16 each, keys permuted within each 32-key
// group to the attention's operand order); otherwise kv is unused. The
// output is fp32 [T][NQ D] in out, or, with out_hi and out_lo (only where
// attn_prefill_uses_split), its bf16 hi and lo split in those two arrays.
bool attn_prefill_uses_split(const Dims& d);
int kv_split_pad(int T);
// causal = false (only where attn_prefill_uses_split): every query sees every key.
// With a split-K workspace (sk) and few query blocks, each block's key range
// is split and the partials merged by a second kernel.
// Q/K-RMSNorm, RoPE and the K/V append of one layer, folded into the prefill
// attention launch (norm = 0: the Q/K rows are used as they are and nothing
// is appended). Rows t are positions pos0 + t.
struct QkRope {
  int norm;
  const float* q_norm;
  const float* k_norm;
  const float* rcos;
  const float* rsin;
  const int64_t* page_table;
  int layer, L, pos0;
  float eps;
};
struct SplitK;
hipError_t launch_attn_prefill(const Dims& d, const float* qkv, int T, float* out, uint16_t* const kv[4],
                               hipStream_t st, uint16_t* out_hi = nullptr, uint16_t* out_lo = nullptr,
                               bool causal = true, SplitK* sk = nullptr, const QkRope* rope = nullptr);
// Whether launch_attn_prefill applies a QkRope itself (else the caller runs
// launch_qk_rope_append first).
bool attn_prefill_ropes(const Dims& d);

hipError_t launch_rms_split(const float* X, int T, int K, const float* gain, float eps, uint16_t* hi,
                            uint16_t* lo, hipStream_t st);
// LayerNorm (population variance, gain and bias) of T rows of K, as bf16 hi/lo
// rows of pitch ldo >= K (0: K) whose columns K .. ldo are zero.
hipError_t launch_ln_split(const float* X, int T, int K, const float* gain, const float* bias, float eps,
                           uint16_t* hi, uint16_t* lo, hipStream_t st, int ldo = 0);
hipError_t launch_rms_apply(const float* X, int T, int K, const float* gain, float eps, float* out,
                            hipStream_t st);
// Workspace of the tiled GEMM's split-K (one per model, adaptor or encoder;
// launches that share one must run on one stream): fp32 partials of C, one
// [M, N] slab per split.
struct SplitK {
  float* P;
  size_t floats;
};
constexpr size_t kSplitKFloats = (size_t)16 << 20;  // 64 MB
// C[M, N] (+)= A[M, K] . W[N, K]^T with a bf16 hi/lo split A (bf16 weights)
// or fp32 A (fp32 weights); the tiled MFMA kernel for M > 64 (with sk, also
// below 128 tiles, splitting K).
// bias (fp32 [N], bf16 weights only) is added to each output before the
// epilogue (STORE, RESID, RELU); nullptr for none.
// With norm set (RESID only), a split launch's reduction also applies the
// next RMSNorm to each finished row and writes it as the next GEMM's bf16
// hi/lo operand (as launch_rms_split would), and sets norm->done; otherwise
// norm->done stays false and the caller runs the norm.
struct RowNorm {
  const float* gain;
  float eps;
  uint16_t* hi;
  uint16_t* lo;
  bool done;
};
hipError_t launch_gemm(bool bf16, Epi epi, const void* A0, const void* A1, int M, int K, const void* W, int N,
                       float* C, int ldc, hipStream_t st, const float* bias = nullptr, SplitK* sk = nullptr,
                       RowNorm* norm = nullptr);
// Whether launch_gemm takes the tiled MFMA kernel for this shape without a
// split-K workspace.
bool gemm_tiled_fits(bool bf16, int M, int K, int N);
// The SwiGLU GEMM on the tiled kernel, its output Z[M, N / 2] (row pitch ldz)
// written as bf16 hi and lo (the down projection's operand); shapes the
// tiled kernel cannot take return hipErrorInvalidValue.
hipError_t launch_gemm_swiglu_split(const uint16_t* A0, const uint16_t* A1, int M, int K, const uint16_t* W, int N,
                                    uint16_t* zhi, uint16_t* zlo, int ldz, hipStream_t st);
hipError_t launch_to_f32(const void* src, bool bf16, size_t n, float* dst, hipStream_t st);

// ---- block-int8 (Q8_0) weights
// A Q8_0 matrix [rows, K] arrives as rows of K / 32 blocks of kQ8BlockBytes:
// an fp16 scale d, then 32 int8 codes q; the weight is q * d. The decode
// kernel reads the codes as int8 rows and the scales from a separate array
// in which each row is cut into segments of kseg inputs (the column slice one
// workgroup's dot covers), each segment's kseg / 32 fp16 scales padded to
// q8_seg_bytes(kseg) bytes so that every segment starts 16-byte aligned.
constexpr int kQ8Block = 32;
constexpr int kQ8BlockBytes = 34;
__host__ __device__ constexpr int q8_seg_bytes(int kseg) { return ((kseg / kQ8Block) * 2 + 15) & ~15; }
// Bytes past the last segment that the decode kernel's 64-byte scale loads
// may read (zero-filled).
constexpr int kQ8ScalePad = 64;
// Unpack rows [0, rows) of a Q8_0 matrix with K inputs per row: source row r
// goes to destination row dst_row(r) = row0 + r, or with gu_half >= 0 to the
// gate/up interleaved row (r / kGuGroup) * 2 kGuGroup + gu_half * kGuGroup +
// r % kGuGroup. Codes to codes[dst_row * K ...], the exact q * d to
// deq[dst_row * K ...] (fp32), scales to the segmented layout at
// scales + (dst_row * (K / kseg) + b / (kseg / 32)) * q8_seg_bytes(kseg).
hipError_t launch_q8_unpack(const void* src, int rows, int K, int kseg, int row0, int gu_half, int8_t* codes,
                            uint16_t* scales, float* deq, hipStream_t st);

// ---- sampling after the LM head (qdec_kernels.hip)
constexpr int kSampleKMax = 128;  // largest top-k
struct SampleUniforms {
  float u[kMaxBatch];
};
// tok[r] for rows r < n of logits [n, V]; hist [n, nh] ids (outside [0, V)
// ignored); temp 0 = greedy (penalty still applied); buf0/buf1 hold
// sample_buffer_words(V) words each.
hipError_t launch_sample(const float* logits, int n, int V, const int32_t* hist, int nh, float rho, float temp,
                         int top_k, float top_p, const SampleUniforms& u, unsigned long long* buf0,
                         unsigned long long* buf1, int32_t* tok, hipStream_t st);
size_t sample_buffer_words(int V);
// The fixed scratch of the allocation-free sampling entry point: both buffers
// on the current device (its address resolved once per device), and the
// largest vocabulary they hold.
hipError_t sample_static_scratch(unsigned long long** buf0, unsigned long long** buf1);
int sample_static_max_vocab();

// ---- audio frontend and SAN-M encoder glue (qdec_encoder.hip)
constexpr int kFrameLen = 400;    // 25 ms at 16 kHz
constexpr int kFrameShift = 160;  // 10 ms
constexpr int kMels = 80;
constexpr double kPreemph = 0.97;
// Float64 tables of the frontend, built on the host: the Hamming window
// [400], FFT twiddles exp(-2 pi i k / 512) for k < 256, and the mel
// triangle weights [80][256] with each filter's nonzero bin range [lo, hi).
struct FrontTables {
  const double* window;
  const double* tw_re;
  const double* tw_im;
  const double* mel_w;
  const int* mel_lo;
  const int* mel_hi;
};
// out[f, 0 .. 80) = log mel energies of frame f, f < n_frames (frame f
// starts at pcm + 160 f; the caller guarantees 400 samples)
hipError_t launch_fbank(const float* pcm, int n_frames, const FrontTables& tb, float* out, hipStream_t st);
// LFR rows [rows, n_mels m] of T frames (lfr, optional) and the encoder input
// rows * scale + sinusoidal positions (x0, optional); inv_freq [n_mels m / 2]
hipError_t launch_lfr_embed(const float* fb, int T, int n_mels, int m, int n, float scale, const double* inv_freq,
                            float* lfr, float* x0, int rows, hipStream_t st);
// out (+)= v + depthwise conv of v over time (v = qkv[:, 2 dim : 3 dim], row
// pitch ld; taps w [dim, K], K odd, zero padding)
hipError_t launch_fsmn(const float* qkv, int ld, int T, int dim, int K, const float* w, bool accumulate, float* out,
                       hipStream_t st);
// LayerNorm (population variance, gain and bias) of T rows of K into fp32;
// out may be X
hipError_t launch_ln_apply(const float* X, int T, int K, const float* gain, const float* bias, float eps, float* out,
                           hipStream_t st);

// ---- persistent decode (qdec_decode.hip)
// Word offsets of the exchange regions inside the model's word buffer.
struct DecOffsets {
  size_t q, att, o, z, x, key, os, xs, att2;
};
// Weight kinds of the decode kernel: the qdec_config weight_dtype codes
// (QDEC_F32, QDEC_BF16, QDEC_Q8_0).
struct DecLaunch {
  Dims d;
  int wt;
  int nblocks;                      // one workgroup per CU, a multiple of 8
  size_t lds_bytes;
  const void* wbuf;                 // packed layer weights, layer l at wbuf + l * layer_elems
  size_t layer_elems, off_o, off_gu, off_d;
  const float* nbuf;                // fp32 norm gains, layer l at nbuf + l * norm_elems
  int norm_elems;
  const void* embed;
  // QDEC_Q8_0: wbuf and embed hold int8 codes; the fp16 scales of layer l
  // start at wscale + l * layer_sbytes (jobs at soff_o, soff_gu, soff_d), the
  // embedding's at escale
  const void* wscale;
  size_t layer_sbytes, soff_o, soff_gu, soff_d;
  const void* escale;
  const float* final_norm;
  const float* rope_cos;
  const float* rope_sin;
  const int64_t* page_table;
  int pos, nsteps, token;
  const int32_t* token_dev;
  float* logits;                    // [nsteps, V] or null
  int32_t* tokens_out;              // [nsteps]
  unsigned long long* ll;           // exchange words
  DecOffsets off;
  unsigned tag0;
  int nsplit_max, whole_max;
  int* err;                         // device address of a host-visible int
  bool local;                       // group-local words at workgroup scope (placement checked)
};
size_t dec_lds_bytes(int wt, const Dims& d, int nblocks, int nsplit_max);
size_t dec_words(const Dims& d, int nblocks, int nsplit_max, DecOffsets* off);
unsigned dec_tags_per_step(const Dims& d);
int dec_split_limit(const Dims& d, int nblocks);
bool dec_fits(int wt, const Dims& d, int nblocks);
hipError_t dec_prepare(int wt, const Dims& d, size_t lds, int* blocks_per_cu);
hipError_t launch_decode(const DecLaunch& a, hipStream_t st);
hipError_t launch_clear_words(unsigned long long* w, size_t n, hipStream_t st);
// Records in out_dev[b] the XCD that workgroup b runs on, for a launch of the
// decode kernel's shape (nblocks x 512 threads, its static LDS plus lds_bytes).
hipError_t launch_xcc_probe(int wt, const Dims& d, int* out_dev, int nblocks, size_t lds_bytes, hipStream_t st);

}  // namespace qdec
