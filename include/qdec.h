/*
 * qdec — Qwen3-0.6B-shaped causal decoder with a paged KV cache, for one
 * AMD Instinct MI355X (gfx950). C ABI: plain pointers and sizes only.
 *
 * What the library computes (cited by page title and section/table):
 *  - audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan", Task 6
 *    Step 4: a Qwen causal decoder with hidden 1024, 28 layers, 16 query and
 *    8 KV heads of dim 128, FFN 3072, RoPE theta 1e6, tied embeddings.
 *  - transcribe.cpp "Forward map - funasr_nano", table "LLM decoder": token
 *    embedding rows, audio rows overriding the span [fbank_beg, +L) of the
 *    input embeddings, 28 blocks of rms_norm + GQA 16/8 + per-head Q/K-RMSNorm
 *    + NeoX RoPE + SwiGLU, a final rms_norm and a tied LM head on the last
 *    position; table "Generation / KV Path": prefill writes the KV cache for
 *    [0, T), then one single-token step per position n_past >= T.
 *  - NCNN "Qwen3ASR ncnn多平台移植", section 5: per step embed, RoPE at the
 *    absolute position, attend over the history plus the current token,
 *    append K/V, full-vocabulary logits, greedy pick; the context holding the
 *    KV cache and position can be cloned to branch from one prefill.
 *
 * Arithmetic: weights bf16, fp32 or block-int8 (QDEC_Q8_0), activations,
 * norms, softmax, logits and the KV cache fp32. RMSNorm is x / sqrt(mean(x^2) + eps) * g. Attention
 * scale is 1/sqrt(head_dim); query head h reads KV head h / (n_q / n_kv).
 * The greedy token is the lowest index among the maximal fp32 logits.
 *
 * Streams: every device operation is enqueued on the HIP stream given to
 * qdec_create; outputs are valid once that stream has been synchronised.
 * Calls are not thread-safe for one model; states of one model share its
 * scratch memory and must be used from one host thread at a time.
 *
 * Errors: every int-returning call returns one of the QDEC_* codes below, and
 * qdec_last_error() returns a description (thread-local, valid until the next
 * call on the same thread). Argument, lifecycle and capacity errors
 * (QDEC_E_INVALID, _POS, _CAPACITY, _STATE) and allocation failures
 * (QDEC_E_OOM) are found before anything is enqueued and leave the state
 * unchanged. QDEC_E_DEVICE from a failed HIP launch may leave the call's
 * earlier launches enqueued (the state's KV pages may then hold partial
 * writes) while the state's position stays unchanged. Device-side waits in
 * the decode and fused GEMM kernels have a time limit; when one expires the
 * kernel still runs to the end, its outputs are invalid, qdec_model_status()
 * reports QDEC_E_DEVICE once the stream has been synchronised, and every
 * later compute call on the model fails with QDEC_E_DEVICE.
 *
 * Device memory: the library's own allocations (packed weights, KV pages,
 * scratch) can be capped for tests with the environment variable
 * QDEC_DEVICE_LIMIT_BYTES, a decimal byte count read at each allocation: an
 * allocation that would take the library's live device bytes past it fails
 * with QDEC_E_OOM as if HBM were full. Memory the caller passes in is not
 * counted. Decode steps after prefill allocate nothing.
 */
#ifndef QDEC_H
#define QDEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDEC_OK 0
#define QDEC_E_INVALID (-1)  /* null pointer, out-of-range argument, bad config */
#define QDEC_E_POS (-2)      /* decode position != n_past */
#define QDEC_E_CAPACITY (-3) /* position or prompt beyond the state's max_ctx */
#define QDEC_E_STATE (-4)    /* wrong lifecycle (prefill on a non-empty state, destroy with live states) */
#define QDEC_E_OOM (-5)      /* device allocation failed */
#define QDEC_E_DEVICE (-6)   /* a HIP runtime error */

/* Weight storage types.
 * QDEC_Q8_0 (audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan",
 * Task 8, which ships Q8_0 weight packages; the page names the type but not
 * its bytes, read here as the common block format): every matrix (WQ, WK, WV,
 * WO, W_GATE, W_UP, W_DOWN and the embedding) is row-major and each row is
 * cut into blocks of 32 consecutive inputs, stored in row order as 34 bytes
 * per block: an IEEE fp16 scale d (little-endian), then 32 int8 codes q. The
 * weight is exactly q * d. The norm gains are fp32. With QDEC_Q8_0 the
 * computation is the same as with fp32 weights equal to q * d: the prefill
 * and batched paths run on that exact dequantization, the single-sequence
 * decode kernel streams the int8 codes and scales (each 32-input partial
 * dot scaled by its block's d). Requires ffn to be a multiple of 256 (each
 * of the 8 slices of W_DOWN's inputs is whole blocks). */
#define QDEC_F32 0
#define QDEC_BF16 1
#define QDEC_Q8_0 2

/* Per-layer tensors, in the order of the qdec_weights.layer table. Linear
 * weights are row-major [out, in]; norm gains are vectors.
 *   IN_NORM [hidden]            input RMSNorm gain
 *   WQ [n_q*hd, hidden]         WK, WV [n_kv*hd, hidden]
 *   Q_NORM, K_NORM [hd]         per-head RMSNorm gains, shared by all heads
 *   WO [hidden, n_q*hd]
 *   POST_NORM [hidden]          post-attention RMSNorm gain
 *   W_GATE, W_UP [ffn, hidden]  W_DOWN [hidden, ffn]
 * The block computes z = silu(W_GATE xn) * (W_UP xn) and x += W_DOWN z. */
enum {
  QDEC_W_IN_NORM = 0,
  QDEC_W_Q,
  QDEC_W_K,
  QDEC_W_V,
  QDEC_W_Q_NORM,
  QDEC_W_K_NORM,
  QDEC_W_O,
  QDEC_W_POST_NORM,
  QDEC_W_GATE,
  QDEC_W_UP,
  QDEC_W_DOWN,
  QDEC_W_PER_LAYER
};

/* Model shape. Validated by qdec_create (QDEC_E_INVALID otherwise):
 * 1 <= n_layer <= 127; hidden a multiple of 64 and <= 1024; head_dim 32, 64
 * or 128; 1 <= n_kv_head <= 8 and n_q_head = 1, 2 or 4 times n_kv_head; ffn a
 * multiple of 64 and <= 8192; n_q_head * head_dim <= 8192; vocab >= 2;
 * rms_eps > 0; rope_theta > 1; each layer's rows per CU fit the decode
 * kernel's LDS staging (true for the Qwen3-0.6B shape on 256 CUs);
 * weight_dtype QDEC_F32, QDEC_BF16 or QDEC_Q8_0; tied == 1 (the LM head is the token
 * embedding table, audio.cpp plan Task 1 Step 3 rejects untied embeddings). */
typedef struct {
  int32_t n_layer, hidden, n_q_head, n_kv_head, head_dim, ffn, vocab;
  float rms_eps, rope_theta;
  int32_t weight_dtype;
  int32_t tied;
} qdec_config;

/* Device pointers to the weights, all of the config's weight_dtype (for
 * QDEC_Q8_0: the matrices as Q8_0 blocks, the norm gains fp32).
 * embed [vocab, hidden] (also the tied LM head), final_norm [hidden].
 * layer: HOST array of n_layer * QDEC_W_PER_LAYER device pointers, layer-major
 * (layer[i * QDEC_W_PER_LAYER + QDEC_W_Q] is layer i's WQ).
 * Ownership: qdec_create copies the per-layer tensors and final_norm into its
 * own packed layout, so those may be freed afterwards; with QDEC_F32 and
 * QDEC_BF16 embed is borrowed and must stay valid until qdec_destroy, with
 * QDEC_Q8_0 it is unpacked into the library's own copies as well. */
typedef struct {
  const void* embed;
  const void* final_norm;
  const void* const* layer;
} qdec_weights;

typedef struct qdec_model qdec_model;
typedef struct qdec_state qdec_state;

/* Validate the config and weights, pack the weights on `hip_stream` (a
 * hipStream_t; NULL = the null stream) and build the RoPE tables. The stream
 * is synchronised before return.
 * The decode kernel exchanges some values only between the workgroups that
 * share one XCD, through that XCD's L2; qdec_create checks with a probe launch
 * that the device places those workgroups together and otherwise exchanges
 * them at device scope. Setting the environment variable
 * QDEC_EXCHANGE_SCOPE=device before qdec_create forces the device-scope form
 * (same results, slower). */
int qdec_create(const qdec_config* cfg, const qdec_weights* w, void* hip_stream, qdec_model** out);

/* Free the model. Returns QDEC_E_STATE (and frees nothing) while states of
 * this model are alive. Synchronises the model's stream. NULL is a no-op. */
int qdec_destroy(qdec_model* m);

/* New empty sequence state (n_past = 0) able to hold max_ctx positions,
 * 1 <= max_ctx <= 1 << 20. Reserves all KV pages now, so decode never
 * allocates. The KV cache is fp32, paged in pages of QDEC_PAGE positions. */
int qdec_state_create(qdec_model* m, int32_t max_ctx, qdec_state** out);
void qdec_state_destroy(qdec_state* s);

#define QDEC_PAGE 16
/* Decode runs at positions below this bound (the decode kernel keeps the
 * state's KV page table on chip); prefill is bounded by max_ctx only. */
#define QDEC_DECODE_MAX_POS 16384

/* Prefill (NCNN page section 5; transcribe.cpp LLM decoder table).
 * ids_host: HOST int32[n_tokens] token ids; ids in [audio_begin,
 *   audio_begin + audio_len) are ignored, all others must lie in [0, vocab).
 * audio_dev: DEVICE fp32 [audio_len, hidden] row-major rows that replace the
 *   token embeddings of that span (may be NULL iff audio_len == 0).
 * Requires n_past == 0 (else QDEC_E_STATE), 1 <= n_tokens <= max_ctx (else
 * QDEC_E_CAPACITY / QDEC_E_INVALID), 0 <= audio_begin, audio_len >= 0,
 * audio_begin + audio_len <= n_tokens.
 * Writes the K/V of positions [0, n_tokens) and sets n_past = n_tokens.
 * logits_dev: DEVICE fp32 [vocab] last-position logits, or NULL.
 * argmax_dev: DEVICE int32 greedy token of the last position, or NULL.
 * Asynchronous: the ids are copied at call time (ids_host may be reused on
 * return); audio_dev must stay valid and outputs are valid once the model's
 * stream has been synchronised. */
int qdec_prefill(qdec_state* s, const int32_t* ids_host, int32_t n_tokens, const float* audio_dev,
                 int32_t audio_begin, int32_t audio_len, float* logits_dev, int32_t* argmax_dev);

/* One decode step (NCNN page section 5, steps 1-6): embeds `token`
 * (0 <= token < vocab), runs all layers at position pos attending over
 * [0, pos], appends K/V at pos and sets n_past = pos + 1.
 * Requires pos == n_past (else QDEC_E_POS), pos < max_ctx and
 * pos < QDEC_DECODE_MAX_POS (else QDEC_E_CAPACITY). logits_dev /
 * argmax_dev as for qdec_prefill. */
int qdec_decode_step(qdec_state* s, int32_t token, int32_t pos, float* logits_dev, int32_t* argmax_dev);

/* As qdec_decode_step, with the token read on the device from token_dev
 * (DEVICE int32, e.g. the previous step's argmax_dev), so greedy decoding
 * needs no host round trip. A token_dev value outside [0, vocab) is clamped
 * into range on the device (the host cannot check it). */
int qdec_decode_step_dev(qdec_state* s, const int32_t* token_dev, int32_t pos, float* logits_dev,
                         int32_t* argmax_dev);

/* n_steps greedy decode steps in one launch (NCNN page section 5: the
 * autoregressive loop of embed, one-token decoder, LM head and pick; section 6:
 * greedy by default). Step 0 consumes *token_dev (DEVICE int32) at position
 * pos; step i > 0 consumes the greedy token of step i-1 at pos + i, without a
 * host round trip. tokens_dev: DEVICE int32 [n_steps], receives each step's
 * greedy token. logits_dev: DEVICE fp32 [n_steps, vocab] or NULL.
 * Requires pos == n_past (else QDEC_E_POS), 1 <= n_steps <= 4096 and
 * pos + n_steps <= min(max_ctx, QDEC_DECODE_MAX_POS) (else QDEC_E_CAPACITY). Sets n_past = pos +
 * n_steps. End-of-sequence handling stays with the caller: every step runs.
 * A *token_dev outside [0, vocab) is clamped into range on the device. */
int qdec_decode_greedy(qdec_state* s, const int32_t* token_dev, int32_t pos, int32_t n_steps, float* logits_dev,
                       int32_t* tokens_dev);

/* n independent decode steps in one launch set (1 <= n <= 16), state i
 * consuming tokens_host[i] at its own n_past. All states must belong to one
 * model and be distinct. Results equal n separate qdec_decode_step calls
 * within rounding. logits_dev: DEVICE fp32 [n, vocab] or NULL; argmax_dev:
 * DEVICE int32 [n] or NULL. On any argument error no state changes. */
int qdec_decode_batch(qdec_state* const* states, int32_t n, const int32_t* tokens_host, float* logits_dev,
                      int32_t* argmax_dev);

/* Clone a state (NCNN page section 5: generation clones the context so one
 * prefill can seed several branches). dst gets src's n_past, max_ctx and a
 * logically identical KV cache: full pages are shared (reference counted,
 * never written again), the partly filled tail page is copied on the stream,
 * and the remaining capacity gets fresh pages. src is unchanged; either may
 * be destroyed first. */
int qdec_clone_state(const qdec_state* src, qdec_state** dst);

/* Sampling options after the LM head (NCNN page section 1: greedy,
 * temperature, top-k, top-p and repetition penalty; section 6: greedy is the
 * default, the others serve non-deterministic generation). */
typedef struct {
  float temperature;         /* 0: greedy (lowest index of the maximum); > 0: sample */
  int32_t top_k;             /* 1 .. QDEC_SAMPLE_TOP_K_MAX when temperature > 0 */
  float top_p;               /* (0, 1]; 1 keeps the whole top-k */
  float repetition_penalty;  /* > 0; 1 is off */
} qdec_sampling;

#define QDEC_SAMPLE_TOP_K_MAX 128

/* Pick one token per row of logits (e.g. from qdec_decode_step or
 * qdec_decode_batch), in this order: every distinct id of the row's history
 * has its logit z divided by repetition_penalty if z > 0, else multiplied by
 * it; greedy when temperature is 0; otherwise z / temperature, candidates
 * ordered by (value descending, index ascending), the first top_k kept,
 * softmax over them, the shortest prefix whose mass reaches top_p kept, and
 * the first candidate whose cumulative mass exceeds uniforms_host[r] times the
 * kept mass is the token. The page gives no formulas; this is the common
 * reading. Values and divisions in float32, the softmax and sums in float64.
 *   logits_dev:    DEVICE fp32 [n_rows, vocab] (borrowed, not modified)
 *   n_rows:        1 .. 16
 *   history_dev:   DEVICE int32 [n_rows, history_len] token ids (ids outside
 *                  [0, vocab) are ignored, e.g. -1 padding); NULL if
 *                  history_len is 0
 *   uniforms_host: HOST fp32 [n_rows], each in [0, 1), supplied by the caller
 *                  (the library draws no random numbers)
 *   tokens_dev:    DEVICE int32 [n_rows], receives the picks
 * Work is enqueued on the model's stream. Errors: QDEC_E_INVALID for bad
 * arguments (top_k outside 1 .. QDEC_SAMPLE_TOP_K_MAX or above vocab with
 * temperature > 0, top_p outside (0, 1], a penalty <= 0, a uniform outside
 * [0, 1), non-finite values), QDEC_E_DEVICE for HIP errors. Non-finite
 * logits give an unspecified token. */
int qdec_sample(qdec_model* m, const float* logits_dev, int32_t n_rows, const qdec_sampling* params,
                const int32_t* history_dev, int32_t history_len, const float* uniforms_host, int32_t* tokens_dev);

/* qdec_sample without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, checks and picks as qdec_sample. Its
 * scratch (the candidate-key buffers) is a fixed 4.9 MB array that the library
 * holds on each GPU it runs on until the process ends; its device address is
 * looked up at qdec_create. That array holds vocabularies of at most
 * QDEC_SAMPLE_NOALLOC_MAX_VOCAB entries (QDEC_E_INVALID for a larger model).
 * All calls on one GPU share the array: calls that overlap on one GPU (for
 * example on two streams) race; calls in sequence on one stream do not. */
#define QDEC_SAMPLE_NOALLOC_MAX_VOCAB 153600
int qdec_sample_noalloc(qdec_model* m, const float* logits_dev, int32_t n_rows, const qdec_sampling* params,
                        const int32_t* history_dev, int32_t history_len, const float* uniforms_host,
                        int32_t* tokens_dev);

/* ---------------------------------------------------------------- adaptor
 * The audio adaptor that makes the rows qdec_prefill takes as audio_dev
 * (transcribe.cpp "Forward map - funasr_nano", section "Adaptor", stage table
 * and its list of deviations from the encoder block): encoder frames
 * [T, enc_dim] -> linear1 + bias -> ReLU -> linear2 + bias -> n_block blocks,
 * each  x += O(MHA(LN1(x)))  with biased Q/K/V/O projections and every frame
 * attending to every frame (scale 1/sqrt(dim / n_head)), then
 * x += fc2(ReLU(fc1(LN2(x))))  with biases. LN(x) = (x - mean) /
 * sqrt(var + ln_eps) * g + b over the row, population variance. The caller
 * keeps the first rows it needs as the prompt's audio span. Weights bf16;
 * activations, norms and softmax fp32. The head count is not on the page:
 * it is a parameter (8 heads of 128 for the 1024-wide adaptor). */
typedef struct {
  int32_t enc_dim;  /* linear1 input, a multiple of 32 */
  int32_t mid_dim;  /* linear1 output, a multiple of 128 */
  int32_t dim;      /* linear2 output and block width, n_head * 128 */
  int32_t ffn_dim;  /* block FFN width, a multiple of 128 */
  int32_t n_block;  /* 1 .. 8 */
  int32_t n_head;   /* heads of 128 */
  float ln_eps;     /* > 0 (1e-12 on the page) */
  int32_t weight_dtype; /* QDEC_BF16 */
} qdec_adaptor_config;

/* Per block, QDEC_AB_PER_BLOCK device pointers in this order; matrices
 * [out, in] row-major, vectors [out]. */
enum {
  QDEC_AB_NORM1_G = 0, QDEC_AB_NORM1_B, QDEC_AB_Q_W, QDEC_AB_Q_B, QDEC_AB_K_W, QDEC_AB_K_B, QDEC_AB_V_W,
  QDEC_AB_V_B, QDEC_AB_O_W, QDEC_AB_O_B, QDEC_AB_NORM2_G, QDEC_AB_NORM2_B, QDEC_AB_FC1_W, QDEC_AB_FC1_B,
  QDEC_AB_FC2_W, QDEC_AB_FC2_B, QDEC_AB_PER_BLOCK
};

/* Device pointers, all bf16: linear1_w [mid_dim, enc_dim], linear1_b
 * [mid_dim], linear2_w [dim, mid_dim], linear2_b [dim]; block: HOST array of
 * n_block * QDEC_AB_PER_BLOCK device pointers, block-major (q/k/v/o [dim,
 * dim], fc1 [ffn_dim, dim], fc2 [dim, ffn_dim]). Ownership: the matrices
 * linear1_w, linear2_w, o, fc1 and fc2 are borrowed and must stay valid until
 * qdec_adaptor_destroy; q/k/v are packed into one [3 dim, dim] copy, and
 * every bias and norm vector is copied (as fp32), so those may be freed. */
typedef struct {
  const void* linear1_w;
  const void* linear1_b;
  const void* linear2_w;
  const void* linear2_b;
  const void* const* block;
} qdec_adaptor_weights;

typedef struct qdec_adaptor qdec_adaptor;

/* Validate (QDEC_E_INVALID), copy and pack on `hip_stream`; the stream is
 * synchronised before return. */
int qdec_adaptor_create(const qdec_adaptor_config* cfg, const qdec_adaptor_weights* w, void* hip_stream,
                        qdec_adaptor** out);

/* Adaptor rows for n_frames encoder frames.
 *   frames_dev: DEVICE fp32 [n_frames, enc_dim] (borrowed, not modified)
 *   n_frames:   >= 1
 *   out_dev:    DEVICE fp32 [n_frames, dim], receives the rows (it also
 *               holds the residual stream while the blocks run, so it must
 *               not overlap frames_dev: QDEC_E_INVALID)
 * Scratch for the largest n_frames seen so far is kept (allocated on first
 * use, QDEC_E_OOM if that fails). Work is enqueued on the adaptor's stream;
 * outputs are valid once it is synchronised. Calls on one adaptor are not
 * thread-safe (they share its scratch). Errors: QDEC_E_INVALID for NULL or
 * undersized buffers, QDEC_E_DEVICE for HIP errors. */
int qdec_adaptor_run(qdec_adaptor* a, const float* frames_dev, int32_t n_frames, float* out_dev);

/* Free the adaptor (synchronises its stream). NULL is a no-op. */
void qdec_adaptor_destroy(qdec_adaptor* a);

/* ------------------------------------------------- frontend and encoder
 * 16 kHz PCM -> log-mel filterbank -> LFR rows -> SAN-M encoder frames, the
 * input of the adaptor.
 * Frontend (audio.cpp "Fun-ASR-Nano Native Runtime Implementation Plan",
 * Task 2 Step 4; transcribe.cpp "Forward map - funasr_nano", table
 * "Frontend"): frames of 400 samples every 160 (whole frames only:
 * T = 1 + (n - 400) / 160); per frame the mean is subtracted, pre-emphasis
 * y[i] = x[i] - 0.97 x[i-1] (y[0] = 0.03 x[0]), Hamming window
 * 0.54 - 0.46 cos(2 pi i / 399), |FFT_512|^2 of bins 0 .. 255, 80 triangle
 * filters on the HTK mel scale 1127 ln(1 + f / 700) with edges equally
 * spaced from 20 to 8000 Hz, natural log floored at the float32 epsilon.
 * LFR row r (ceil(T / lfr_n) rows) stacks frames
 * clamp(r lfr_n + j - (lfr_m - 1) / 2, 0, T - 1), j < lfr_m. No CMVN.
 * Encoder (same plan, Tasks 3-4; the map's "Encoder" table): x = LFR rows *
 * sqrt(dim) + PE (PE[t, 2i] = sin(t / 10000^(2i/W)), PE[t, 2i+1] = cos, W =
 * the row width); then 1 + n_main + n_tp SAN-M blocks, each
 *   h = LN1(x); q, k, v = h Wq + bq, h Wk + bk, h Wv + bv;
 *   y = MHA(q, k, v) Wo + bo + v + fsmn(v)   (every frame sees every frame,
 *       scale 1/sqrt(128); fsmn = per-channel conv over time with K taps,
 *       zero padding (K-1)/2 each side, no bias);
 *   x = x + y (the first block, the 560 -> dim stem: x = y);
 *   x = x + W2 ReLU(W1 LN2(x) + b1) + b2,
 * with LN = after_norm applied after block n_main and LN = tp_norm after the
 * last; LN(x) = (x - mean) / sqrt(var + ln_eps) g + b, population variance.
 * Frontend in float64, encoder weights bf16 with fp32 activations. Head
 * count, FFN width and FSMN taps are not given by the pages for the real
 * encoder: parameters (4 heads, 2048, 11 in the workloads). */
typedef struct {
  int32_t n_mels;       /* 80 */
  int32_t lfr_m;        /* frames per LFR row, odd, 1 .. 15 (7) */
  int32_t lfr_n;        /* LFR stride in frames, 1 .. 15 (6) */
  int32_t dim;          /* n_head * 128 */
  int32_t n_head;
  int32_t ffn_dim;      /* a multiple of 128 */
  int32_t fsmn_kernel;  /* odd, 1 .. 31 */
  int32_t n_main;       /* residual blocks after the stem, 0 .. 127 (49) */
  int32_t n_tp;         /* blocks after after_norm, 0 .. 127 (20) */
  float ln_eps;         /* > 0 (1e-12) */
  int32_t weight_dtype; /* QDEC_BF16 */
} qdec_encoder_config;

/* Per block, QDEC_EB_PER_BLOCK device pointers in this order; matrices
 * [out, in] row-major, vectors [out]; the stem's norm1 and q/k/v take
 * in = n_mels * lfr_m inputs, every other block in = dim. FSMN taps
 * [dim, fsmn_kernel]. */
enum {
  QDEC_EB_NORM1_G = 0, QDEC_EB_NORM1_B, QDEC_EB_Q_W, QDEC_EB_Q_B, QDEC_EB_K_W, QDEC_EB_K_B, QDEC_EB_V_W,
  QDEC_EB_V_B, QDEC_EB_FSMN_W, QDEC_EB_O_W, QDEC_EB_O_B, QDEC_EB_NORM2_G, QDEC_EB_NORM2_B, QDEC_EB_FFN1_W,
  QDEC_EB_FFN1_B, QDEC_EB_FFN2_W, QDEC_EB_FFN2_B, QDEC_EB_PER_BLOCK
};

/* Device pointers, all bf16: block: HOST array of (1 + n_main + n_tp) *
 * QDEC_EB_PER_BLOCK device pointers, block-major in run order (stem, main
 * blocks, tp blocks); after_norm and tp_norm gains and biases [dim].
 * Ownership: o, ffn1 and ffn2 are borrowed and must stay valid until
 * qdec_encoder_destroy; q/k/v are packed into one [3 dim, in] copy (the
 * stem's columns padded to a multiple of 32), taps and vectors are copied as
 * fp32, so those may be freed. */
typedef struct {
  const void* const* block;
  const void* after_norm_g;
  const void* after_norm_b;
  const void* tp_norm_g;
  const void* tp_norm_b;
} qdec_encoder_weights;

typedef struct qdec_encoder qdec_encoder;

/* Validate (QDEC_E_INVALID), copy, pack and build the frontend tables on
 * `hip_stream`; the stream is synchronised before return. */
int qdec_encoder_create(const qdec_encoder_config* cfg, const qdec_encoder_weights* w, void* hip_stream,
                        qdec_encoder** out);

/* LFR rows for n_samples of PCM: ceil(T / lfr_n), T = 1 + (n_samples - 400)
 * / 160 whole frames; 0 below 400 samples or for a NULL encoder. */
int32_t qdec_encoder_rows(const qdec_encoder* e, int64_t n_samples);

/* Frontend only: lfr_dev DEVICE fp32 [rows, n_mels * lfr_m] receives the LFR
 * rows of pcm_dev (DEVICE fp32 [n_samples], at least 400 samples, else
 * QDEC_E_INVALID). */
int qdec_frontend_run(qdec_encoder* e, const float* pcm_dev, int64_t n_samples, float* lfr_dev);

/* Encoder only: out_dev DEVICE fp32 [n_rows, dim] receives the encoder
 * frames (tp_norm's output) of lfr_dev (DEVICE fp32 [n_rows, n_mels *
 * lfr_m], n_rows >= 1, not modified). */
int qdec_encoder_forward(qdec_encoder* e, const float* lfr_dev, int32_t n_rows, float* out_dev);

/* Both: out_dev DEVICE fp32 [qdec_encoder_rows(e, n_samples), dim]. */
int qdec_encoder_run(qdec_encoder* e, const float* pcm_dev, int64_t n_samples, float* out_dev);

/* Scratch for the longest input seen so far is kept (QDEC_E_OOM if it cannot
 * grow). Work is enqueued on the encoder's stream; calls on one encoder are
 * not thread-safe. Errors: QDEC_E_INVALID for NULL or undersized buffers,
 * QDEC_E_DEVICE for HIP errors. Free with qdec_encoder_destroy (synchronises
 * its stream; NULL is a no-op). */
void qdec_encoder_destroy(qdec_encoder* e);

/* n_past of the state (-1 for NULL). */
int32_t qdec_state_pos(const qdec_state* s);

/* QDEC_OK, or QDEC_E_DEVICE if a device-side wait of any launch on this model
 * has hit its time limit (the outputs of that launch and of later ones are
 * invalid and the model must be recreated). Call it after synchronising the
 * model's stream to confirm the outputs of asynchronous calls; QDEC_E_INVALID
 * for NULL. */
int qdec_model_status(const qdec_model* m);

/* Description of the last error on this thread ("" if none). */
const char* qdec_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QDEC_H */
