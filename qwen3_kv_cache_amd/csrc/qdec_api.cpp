// Host side of the qdec C ABI: argument validation, weight packing, the
// paged KV pool with reference-counted pages, sequence states and launch
// sequencing. Everything device-side is enqueued on the model's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "qdec_internal.h"

using namespace qdec;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return QDEC_OK;
}

// Every device allocation of the library goes through dmalloc / dfree, which
// keep the number of live bytes. The environment variable
// QDEC_DEVICE_LIMIT_BYTES, read at each allocation, caps that number: an
// allocation that would pass it fails as hipMalloc does when HBM is full, so a
// test can reach every QDEC_E_OOM path on a GPU with memory to spare.
std::mutex g_mem_mu;
std::unordered_map<void*, size_t> g_mem_live;
size_t g_mem_bytes = 0;

hipError_t dmalloc_bytes(void** p, size_t bytes) {
  *p = nullptr;
  std::lock_guard<std::mutex> lock(g_mem_mu);
  if (const char* lim = getenv("QDEC_DEVICE_LIMIT_BYTES")) {
    char* end = nullptr;
    const unsigned long long cap = strtoull(lim, &end, 10);
    if (end != lim && *end == '\0' && (bytes > cap || g_mem_bytes > cap - bytes)) return hipErrorOutOfMemory;
  }
  const hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return e;
  }
  if (*p) {
    g_mem_live[*p] = bytes;
    g_mem_bytes += bytes;
  }
  return hipSuccess;
}

template <typename T>
hipError_t dmalloc(T** p, size_t bytes) {
  return dmalloc_bytes((void**)p, bytes);
}

hipError_t dfree(void* p) {
  if (!p) return hipSuccess;
  {
    std::lock_guard<std::mutex> lock(g_mem_mu);
    auto it = g_mem_live.find(p);
    if (it != g_mem_live.end()) {
      g_mem_bytes -= it->second;
      g_mem_live.erase(it);
    }
  }
  return hipFree(p);
}

#define HIP_TRY(expr)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(QDEC_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Checks that [p, p + bytes) lies inside one device allocation, so a kernel
// never writes or reads past what the caller handed in.
int check_dev(const void* p, size_t bytes, const char* what) {
  if (!p) return fail(QDEC_E_INVALID, "%s is NULL", what);
  hipPointerAttribute_t attr;
  const hipError_t pe = hipPointerGetAttributes(&attr, p);
  if (pe != hipSuccess) {
    (void)hipGetLastError();
    return fail(QDEC_E_INVALID, "%s is not a device pointer (%s)", what, hipGetErrorString(pe));
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(QDEC_E_INVALID, "%s is not device memory", what);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(QDEC_E_INVALID, "%s: cannot query its allocation", what);
  }
  const char* b = (const char*)base;
  const char* q = (const char*)p;
  if (q < b || q + bytes > b + size)
    return fail(QDEC_E_INVALID, "%s: %zu bytes do not fit its allocation", what, bytes);
  return QDEC_OK;
}

struct PagePool {
  size_t page_bytes = 0;
  std::vector<void*> chunks;
  std::vector<char*> free_pages;
  std::unordered_map<char*, int> refs;

  int reserve(int n) {
    if ((int)free_pages.size() >= n) return QDEC_OK;
    const int want = n - (int)free_pages.size();
    const int npages = want < 32 ? 32 : want;
    void* p = nullptr;
    if (dmalloc(&p, (size_t)npages * page_bytes) != hipSuccess) {
      (void)hipGetLastError();
      return fail(QDEC_E_OOM, "KV pool: cannot allocate %d pages of %zu bytes", npages, page_bytes);
    }
    chunks.push_back(p);
    for (int i = npages - 1; i >= 0; --i) free_pages.push_back((char*)p + (size_t)i * page_bytes);
    return QDEC_OK;
  }
  char* take() {
    char* p = free_pages.back();
    free_pages.pop_back();
    refs[p] = 1;
    return p;
  }
  void retain(char* p) { ++refs[p]; }
  void release(char* p) {
    auto it = refs.find(p);
    if (it == refs.end()) return;
    if (--it->second == 0) {
      refs.erase(it);
      free_pages.push_back(p);
    }
  }
};

template <typename T>
int dev_alloc(T** p, size_t n, const char* what) {
  *p = nullptr;
  if (n == 0) return QDEC_OK;
  if (dmalloc((void**)p, n * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(QDEC_E_OOM, "cannot allocate %s (%zu bytes)", what, n * sizeof(T));
  }
  return QDEC_OK;
}

// A split-K workspace for the tiled GEMM (kSplitKFloats fp32 partials).
struct SplitKBuf {
  SplitK sk{nullptr, 0};
};
int alloc_splitk(SplitKBuf* b) {
  if (int e = dev_alloc(&b->sk.P, kSplitKFloats, "split-K partials")) return e;
  b->sk.floats = kSplitKFloats;
  return QDEC_OK;
}
void free_splitk(SplitKBuf* b) {
  (void)dfree(b->sk.P);
  b->sk.P = nullptr;
}

}  // namespace

struct qdec_model {
  qdec_config cfg{};
  Dims d{};
  bool bf16 = true;  // bf16 weights in wbuf / embed (else fp32)
  int wt = QDEC_BF16;  // the config's weight_dtype
  // QDEC_Q8_0: wbuf and embed hold the exactly dequantized fp32 weights (the
  // prefill and batched paths); the decode kernel streams int8 codes and the
  // segmented fp16 scales below
  int8_t* q_codes = nullptr;
  uint16_t* q_scales = nullptr;
  int8_t* q_embed = nullptr;
  uint16_t* q_escale = nullptr;
  float* embed_own = nullptr;
  size_t layer_sbytes = 0, soff_o = 0, soff_gu = 0, soff_d = 0;
  hipStream_t stream = nullptr;
  const void* embed = nullptr;
  float* final_norm = nullptr;
  void* wbuf = nullptr;  // packed matrices of all layers
  float* nbuf = nullptr; // fp32 norm gains of all layers
  std::vector<LayerW> layers;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  int rope_cap = 0;
  unsigned long long* keys = nullptr;  // prefill argmax key
  int32_t* argmax_tmp = nullptr;
  // prefill scratch, grown on demand
  int pf_cap = 0;
  int32_t* p_ids = nullptr;
  float* pX = nullptr;
  float* pQKV = nullptr;
  float* pAttn = nullptr;
  uint16_t* pKV[4] = {nullptr, nullptr, nullptr, nullptr};  // converted K / V^T for the matrix-core attention
  float* pZ = nullptr;
  void* pA0 = nullptr;  // bf16 hi (or fp32 activations for fp32 weights)
  void* pA1 = nullptr;  // bf16 lo
  // batched decode workspace for kMaxBatch rows, allocated on first use
  bool b_ready = false;
  float* bX = nullptr;
  float* bQKV = nullptr;
  float* bAttn = nullptr;
  float* bZ = nullptr;
  void* bA0 = nullptr;
  void* bA1 = nullptr;
  float* bLogits = nullptr;  // logits when the caller passes none
  unsigned long long* bKeys = nullptr;
  int32_t* bTok = nullptr;   // argmax when the caller passes none
  unsigned long long* bAttnPart = nullptr;  // split partial words of batched attention
  unsigned* bAttnCnt = nullptr;
  int b_nsplit_cap = 0;
  // fused small-M GEMM workspace (up to 64 rows): split-K partials, arrival
  // counters, RMSNorm sum-of-squares partials
  unsigned long long* rP = nullptr;
  size_t rP_words = 0;
  unsigned rows_tag = 1;  // tag of the next fused GEMM launch
  unsigned* rCnt = nullptr;
  float* rSsq = nullptr;
  // sampling workspace: two candidate-key buffers
  unsigned long long* sBuf0 = nullptr;
  unsigned long long* sBuf1 = nullptr;
  // the same for qdec_sample_noalloc: the device's fixed scratch array
  unsigned long long* sStatic0 = nullptr;
  unsigned long long* sStatic1 = nullptr;
  PagePool pool;
  int live_states = 0;
  // persistent decode
  int dec_blocks = 0;
  size_t dec_lds = 0;
  int nsplit_max = 1, whole_max = 64;
  unsigned long long* ll = nullptr;
  size_t ll_words = 0;
  DecOffsets off{};
  unsigned tag_next = 1;  // next unused exchange tag (0 marks a cleared word)
  int* err_host = nullptr;
  int* err_dev = nullptr;
  bool dec_local = false;  // decode kernel's group-local words at workgroup scope
  // pinned host staging for asynchronous uploads (prompt ids, page tables):
  // a buffer is rewritten only after the event of its last copy has completed
  struct Staging {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
  } st_ids, st_pt;
  size_t layer_elems = 0, off_o = 0, off_gu = 0, off_d = 0;
  int norm_elems = 0;
  SplitKBuf split;  // the prefill GEMMs' split-K workspace
};

struct qdec_state {
  qdec_model* m = nullptr;
  int max_ctx = 0;
  int n_past = 0;
  std::vector<char*> pages;
  int64_t* pt_dev = nullptr;
};

namespace {

int validate_config(const qdec_config* c) {
  if (!c) return fail(QDEC_E_INVALID, "config is NULL");
  if (c->n_layer < 1 || c->n_layer > 127) return fail(QDEC_E_INVALID, "n_layer %d out of range", c->n_layer);
  if (c->hidden < 64 || c->hidden > 1024 || c->hidden % 64)
    return fail(QDEC_E_INVALID, "hidden %d must be a multiple of 64 in [64, 1024]", c->hidden);
  if (c->head_dim < 8 || c->head_dim > 128 || c->head_dim % 8)
    return fail(QDEC_E_INVALID, "head_dim %d must be a multiple of 8 in [8, 128]", c->head_dim);
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(QDEC_E_INVALID, "head_dim %d: kernels are built for 32, 64 and 128", c->head_dim);
  if (c->n_kv_head < 1 || c->n_q_head < c->n_kv_head || c->n_q_head % c->n_kv_head)
    return fail(QDEC_E_INVALID, "n_q_head %d must be a positive multiple of n_kv_head %d", c->n_q_head,
                c->n_kv_head);
  const int group = c->n_q_head / c->n_kv_head;
  if (group != 1 && group != 2 && group != 4)
    return fail(QDEC_E_INVALID, "GQA group %d must be 1, 2 or 4", group);
  if (c->n_kv_head > 8) return fail(QDEC_E_INVALID, "n_kv_head %d > 8", c->n_kv_head);
  if (c->n_q_head * c->head_dim > 8192) return fail(QDEC_E_INVALID, "n_q_head * head_dim exceeds 8192");
  if (c->ffn < 64 || c->ffn > 8192 || c->ffn % 64)
    return fail(QDEC_E_INVALID, "ffn %d must be a multiple of 64 in [64, 8192]", c->ffn);
  if (c->vocab < 2) return fail(QDEC_E_INVALID, "vocab %d < 2", c->vocab);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(QDEC_E_INVALID, "rms_eps must be > 0");
  if (!(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta))
    return fail(QDEC_E_INVALID, "rope_theta must be > 1");
  if (c->weight_dtype != QDEC_F32 && c->weight_dtype != QDEC_BF16 && c->weight_dtype != QDEC_Q8_0)
    return fail(QDEC_E_INVALID, "weight_dtype %d unknown", c->weight_dtype);
  if (c->weight_dtype == QDEC_Q8_0 && c->ffn % (8 * kQ8Block))
    return fail(QDEC_E_INVALID, "Q8_0 weights need ffn %d to be a multiple of %d", c->ffn, 8 * kQ8Block);
  if (c->tied != 1) return fail(QDEC_E_INVALID, "untied LM head is not supported (tied must be 1)");
  return QDEC_OK;
}

void free_prefill(qdec_model* m) {
  (void)dfree(m->p_ids);
  (void)dfree(m->pX);
  (void)dfree(m->pQKV);
  (void)dfree(m->pAttn);
  for (uint16_t*& p : m->pKV) {
    (void)dfree(p);
    p = nullptr;
  }
  (void)dfree(m->pZ);
  (void)dfree(m->pA0);
  (void)dfree(m->pA1);
  m->p_ids = nullptr;
  m->pX = m->pQKV = m->pAttn = m->pZ = nullptr;
  m->pA0 = m->pA1 = nullptr;
  m->pf_cap = 0;
}

void free_batch(qdec_model* m) {
  for (void* p : {(void*)m->bX, (void*)m->bQKV, (void*)m->bAttn, (void*)m->bZ, m->bA0, m->bA1,
                  (void*)m->bLogits, (void*)m->bKeys, (void*)m->bTok, (void*)m->bAttnPart, (void*)m->bAttnCnt})
    (void)dfree(p);
  m->bX = m->bQKV = m->bAttn = m->bZ = m->bLogits = nullptr;
  m->bAttnPart = nullptr;
  m->bAttnCnt = nullptr;
  m->bA0 = m->bA1 = nullptr;
  m->bKeys = nullptr;
  m->bTok = nullptr;
  m->b_nsplit_cap = 0;
  m->b_ready = false;
}

void free_model(qdec_model* m) {
  if (!m) return;
  if (m->stream) (void)hipStreamSynchronize(m->stream);
  free_batch(m);
  (void)dfree(m->rP);
  (void)dfree(m->rCnt);
  (void)dfree(m->rSsq);
  (void)dfree(m->sBuf0);
  (void)dfree(m->sBuf1);
  (void)dfree(m->final_norm);
  (void)dfree(m->wbuf);
  (void)dfree(m->q_codes);
  (void)dfree(m->q_scales);
  (void)dfree(m->q_embed);
  (void)dfree(m->q_escale);
  (void)dfree(m->embed_own);
  (void)dfree(m->nbuf);
  (void)dfree(m->rope_cos);
  (void)dfree(m->rope_sin);
  (void)dfree(m->keys);
  (void)dfree(m->argmax_tmp);
  free_prefill(m);
  (void)dfree(m->ll);
  free_splitk(&m->split);
  if (m->err_host) (void)hipHostFree(m->err_host);
  for (qdec_model::Staging* g : {&m->st_ids, &m->st_pt}) {
    if (g->host) (void)hipHostFree(g->host);
    if (g->ev) (void)hipEventDestroy(g->ev);
  }
  for (void* c : m->pool.chunks) (void)dfree(c);
  delete m;
}

int ensure_rope(qdec_model* m, int n_pos) {
  if (n_pos <= m->rope_cap) return QDEC_OK;
  int cap = m->rope_cap ? m->rope_cap : 1024;
  while (cap < n_pos) cap *= 2;
  const int half = m->d.D / 2;
  std::vector<float> c((size_t)cap * half), s((size_t)cap * half);
  // angle = p * theta^(-2j/D) in double precision, then rounded to float
  std::vector<double> freq(half);
  for (int j = 0; j < half; ++j) freq[j] = std::pow((double)m->cfg.rope_theta, -2.0 * j / m->d.D);
  for (int p = 0; p < cap; ++p)
    for (int j = 0; j < half; ++j) {
      const double a = (double)p * freq[j];
      c[(size_t)p * half + j] = (float)std::cos(a);
      s[(size_t)p * half + j] = (float)std::sin(a);
    }
  float *dc = nullptr, *ds = nullptr;
  if (int e = dev_alloc(&dc, c.size(), "RoPE table")) return e;
  if (int e = dev_alloc(&ds, s.size(), "RoPE table")) {
    (void)dfree(dc);
    return e;
  }
  HIP_TRY(hipMemcpy(dc, c.data(), c.size() * sizeof(float), hipMemcpyHostToDevice));
  HIP_TRY(hipMemcpy(ds, s.data(), s.size() * sizeof(float), hipMemcpyHostToDevice));
  // older tables may still be read by queued work
  HIP_TRY(hipStreamSynchronize(m->stream));
  (void)dfree(m->rope_cos);
  (void)dfree(m->rope_sin);
  m->rope_cos = dc;
  m->rope_sin = ds;
  m->rope_cap = cap;
  return QDEC_OK;
}

int ensure_prefill(qdec_model* m, int T) {
  if (T <= m->pf_cap) return QDEC_OK;
  HIP_TRY(hipStreamSynchronize(m->stream));
  free_prefill(m);
  const Dims& d = m->d;
  const int kmax = std::max(std::max(d.H, d.NQ * d.D), d.F);
  int e = 0;
  if ((e = dev_alloc(&m->p_ids, T, "prefill ids")) || (e = dev_alloc(&m->pX, (size_t)T * d.H, "prefill X")) ||
      (e = dev_alloc(&m->pQKV, (size_t)T * d.qkv(), "prefill QKV")) ||
      (e = dev_alloc(&m->pAttn, (size_t)T * d.NQ * d.D, "prefill attention")) ||
      (attn_prefill_uses_split(d) &&
       ((e = dev_alloc(&m->pKV[0], (size_t)d.NKV * T * d.D, "prefill K")) ||
        (e = dev_alloc(&m->pKV[1], (size_t)d.NKV * T * d.D, "prefill K")) ||
        (e = dev_alloc(&m->pKV[2], (size_t)d.NKV * d.D * kv_split_pad(T), "prefill V")) ||
        (e = dev_alloc(&m->pKV[3], (size_t)d.NKV * d.D * kv_split_pad(T), "prefill V")))) ||
      (e = dev_alloc(&m->pZ, (size_t)T * d.F, "prefill FFN"))) {
    free_prefill(m);
    return e;
  }
  const size_t abytes = m->bf16 ? 2 : 4;
  if (dmalloc(&m->pA0, (size_t)T * kmax * abytes) != hipSuccess ||
      (m->bf16 && dmalloc(&m->pA1, (size_t)T * kmax * abytes) != hipSuccess)) {
    (void)hipGetLastError();
    free_prefill(m);
    return fail(QDEC_E_OOM, "cannot allocate prefill activations for %d tokens", T);
  }
  m->pf_cap = T;
  return QDEC_OK;
}

// ---------------------------------------------------------------- passes

#define LAUNCH(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(QDEC_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// One launch of `nsteps` greedy decode steps of one sequence; the state's
// n_past is updated by the caller.
int run_decode(qdec_state* s, int token, const int32_t* token_dev, int pos, int nsteps, float* logits,
               int32_t* tokens_out) {
  qdec_model* m = s->m;
  const Dims& d = m->d;
  hipStream_t st = m->stream;
  if (__atomic_load_n(m->err_host, __ATOMIC_ACQUIRE))
    return fail(QDEC_E_DEVICE, "an earlier launch hit its time limit; the model must be recreated");
  if ((int64_t)pos + nsteps > kDecMaxPos)
    return fail(QDEC_E_CAPACITY, "decode reaches position %lld; decode supports positions below %d",
                (long long)pos + nsteps - 1, kDecMaxPos);
  // tags never repeat while stale words could still hold them: before the
  // counter would wrap, every word is cleared and tags restart at 1
  const unsigned need = (unsigned)nsteps * dec_tags_per_step(d);
  if (m->tag_next + (unsigned long long)need >= 0x7FFFFFFFull) {
    LAUNCH(launch_clear_words(m->ll, m->ll_words, st));
    m->tag_next = 1;
  }
  DecLaunch a{};
  a.d = d;
  a.wt = m->wt;
  a.nblocks = m->dec_blocks;
  a.lds_bytes = m->dec_lds;
  const bool q8 = m->wt == QDEC_Q8_0;
  a.wbuf = q8 ? (const void*)m->q_codes : m->wbuf;
  a.layer_elems = m->layer_elems;
  a.off_o = m->off_o;
  a.off_gu = m->off_gu;
  a.off_d = m->off_d;
  a.nbuf = m->nbuf;
  a.norm_elems = m->norm_elems;
  a.embed = q8 ? (const void*)m->q_embed : m->embed;
  a.wscale = m->q_scales;
  a.layer_sbytes = m->layer_sbytes;
  a.soff_o = m->soff_o;
  a.soff_gu = m->soff_gu;
  a.soff_d = m->soff_d;
  a.escale = m->q_escale;
  a.final_norm = m->final_norm;
  a.rope_cos = m->rope_cos;
  a.rope_sin = m->rope_sin;
  a.page_table = s->pt_dev;
  a.pos = pos;
  a.nsteps = nsteps;
  a.token = token;
  a.token_dev = token_dev;
  a.logits = logits;
  a.tokens_out = tokens_out ? tokens_out : m->argmax_tmp;
  a.ll = m->ll;
  a.off = m->off;
  a.tag0 = m->tag_next;
  a.nsplit_max = m->nsplit_max;
  a.whole_max = m->whole_max;
  a.err = m->err_dev;
  a.local = m->dec_local;
  LAUNCH(launch_decode(a, st));
  m->tag_next += need;
  return QDEC_OK;
}

int ensure_batch(qdec_model* m, int nsplit) {
  const Dims& d = m->d;
  constexpr int B = kMaxBatch;
  if (!m->b_ready) {
    const int kmax = std::max(std::max(d.H, d.NQ * d.D), d.F);
    const size_t abytes = m->bf16 ? 2 : 4;
    int e = 0;
    if ((e = dev_alloc(&m->bX, (size_t)B * d.H, "batch X")) ||
        (e = dev_alloc(&m->bQKV, (size_t)B * d.qkv(), "batch QKV")) ||
        (e = dev_alloc(&m->bAttn, (size_t)B * d.NQ * d.D, "batch attention")) ||
        (e = dev_alloc(&m->bZ, (size_t)B * d.F, "batch FFN")) ||
        (e = dev_alloc(&m->bLogits, (size_t)B * d.V, "batch logits")) ||
        (e = dev_alloc(&m->bKeys, (size_t)B * kKeySlots, "batch keys")) || (e = dev_alloc(&m->bTok, (size_t)B, "batch tokens")) ||
        (e = dev_alloc(&m->bAttnCnt, (size_t)B * d.NKV, "batch attention counters"))) {
      free_batch(m);
      return e;
    }
    if (dmalloc(&m->bA0, (size_t)B * kmax * abytes) != hipSuccess ||
        (m->bf16 && dmalloc(&m->bA1, (size_t)B * kmax * abytes) != hipSuccess)) {
      (void)hipGetLastError();
      free_batch(m);
      return fail(QDEC_E_OOM, "cannot allocate batch activations");
    }
    HIP_TRY(hipMemset(m->bAttnCnt, 0, (size_t)B * d.NKV * sizeof(unsigned)));
    m->b_ready = true;
  }
  if (nsplit > m->b_nsplit_cap) {
    HIP_TRY(hipStreamSynchronize(m->stream));
    (void)dfree(m->bAttnPart);
    m->bAttnPart = nullptr;
    m->b_nsplit_cap = 0;
    const size_t words = (size_t)B * d.NQ * nsplit * (d.D + 2);
    if (int e = dev_alloc(&m->bAttnPart, words, "batch attention partials")) return e;
    HIP_TRY(hipMemset(m->bAttnPart, 0, words * sizeof(unsigned long long)));  // tag 0 is never used
    m->b_nsplit_cap = nsplit;
  }
  return QDEC_OK;
}

// Workspace of the fused small-M GEMMs, sized for 64 rows; counters start at
// zero and every launch leaves them at zero.
int ensure_rows(qdec_model* m) {
  if (m->rP) return QDEC_OK;
  const Dims& d = m->d;
  constexpr int R = 64;
  const int shapes[5][2] = {{d.H, d.qkv()}, {d.NQ * d.D, d.H}, {d.H, 2 * d.F}, {d.F, d.H}, {d.H, d.V}};
  size_t part = 1;
  int cnt = 1;
  // the split depends on the row count: the largest need over 1 .. R rows
  for (auto& kn : shapes) {
    for (int M = 1; M <= R; ++M) {
      if (!rows_fits(M, kn[0], kn[1])) continue;
      part = std::max(part, rows_partial_floats(M, kn[0], kn[1]));
      cnt = std::max(cnt, rows_counters(M, kn[0], kn[1]));
    }
  }
  const size_t nss = (size_t)std::max(1, d.H / 16);
  int e = 0;
  if ((e = dev_alloc(&m->rP, part, "GEMM partial tiles")) || (e = dev_alloc(&m->rCnt, (size_t)cnt, "GEMM counters")) ||
      (e = dev_alloc(&m->rSsq, nss * R, "RMSNorm partials"))) {
    (void)dfree(m->rP);
    (void)dfree(m->rCnt);
    (void)dfree(m->rSsq);
    m->rP = nullptr;
    m->rSsq = nullptr;
    m->rCnt = nullptr;
    return e;
  }
  HIP_TRY(hipMemset(m->rCnt, 0, (size_t)cnt * sizeof(unsigned)));
  HIP_TRY(hipMemset(m->rP, 0, part * sizeof(unsigned long long)));
  m->rP_words = part;
  m->rows_tag = 1;
  return QDEC_OK;
}

// Tag for the next fused GEMM launch. Before the counter would wrap, the
// partial words are cleared (tag 0 is never used), so no stale word can match.
int next_rows_tag(qdec_model* m, unsigned* tag) {
  if (m->rows_tag >= 0xFFFFFFF0u) {
    if (m->rP) HIP_TRY(hipMemsetAsync(m->rP, 0, m->rP_words * sizeof(unsigned long long), m->stream));
    if (m->bAttnPart)
      HIP_TRY(hipMemsetAsync(m->bAttnPart, 0,
                             (size_t)kMaxBatch * m->d.NQ * m->b_nsplit_cap * (m->d.D + 2) * sizeof(unsigned long long),
                             m->stream));
    m->rows_tag = 1;
  }
  *tag = m->rows_tag++;
  return QDEC_OK;
}

int gemm_rows(qdec_model* m, Epi epi, bool norm, RowsGemm& g) {
  if (int e = next_rows_tag(m, &g.tag)) return e;
  g.wf32 = m->bf16 ? 0 : 1;
  g.err = m->err_dev;
  LAUNCH(launch_gemm_rows(epi, norm, g, m->stream));
  return QDEC_OK;
}

bool use_rows(const qdec_model* m, int T) {
  const Dims& d = m->d;
  return rows_fits(T, d.H, d.qkv()) && rows_fits(T, d.NQ * d.D, d.H) && rows_fits(T, d.H, 2 * d.F) &&
         rows_fits(T, d.F, d.H);
}

// The decoder layers over T <= 64 rows with the fused GEMMs: RMSNorm runs in
// the prologue of the GEMM that consumes it (from sum-of-squares partials the
// producer left in rSsq, nss of them per row), residual adds and SwiGLU in the
// epilogues. Returns the partial count per row of the final X in *nss_out.
template <typename RopeFn, typename AttnFn>
int run_layers_rows(qdec_model* m, int T, float* X, float* QKV, float* Attn, float* Z, int nss, RopeFn rope,
                    AttnFn attn, int* nss_out) {
  const Dims& d = m->d;
  RowsGemm g{};
  g.M = T;
  g.eps = d.eps;
  g.P = m->rP;
  g.cnt = m->rCnt;
  const int nss_h = d.H / rows_tile_cols(d.H);
  for (int l = 0; l < d.L; ++l) {
    const LayerW& w = m->layers[l];
    g.A = X, g.lda = d.H, g.ssq = m->rSsq, g.nss = nss, g.gain = w.in_norm;
    g.W = w.wqkv, g.K = d.H, g.N = d.qkv(), g.C = QKV, g.ldc = d.qkv();
    if (int e = gemm_rows(m, EPI_STORE, true, g)) return e;
    if (int e = rope(l)) return e;
    if (int e = attn(l, nullptr, nullptr)) return e;
    g.A = Attn, g.lda = d.NQ * d.D, g.W = w.wo, g.K = d.NQ * d.D, g.N = d.H, g.C = X, g.ldc = d.H;
    g.ssq_out = m->rSsq;
    if (int e = gemm_rows(m, EPI_RESID, false, g)) return e;
    g.A = X, g.lda = d.H, g.ssq = m->rSsq, g.nss = nss_h, g.gain = w.post_norm;
    g.W = w.wgu, g.K = d.H, g.N = 2 * d.F, g.C = Z, g.ldc = d.F;
    if (int e = gemm_rows(m, EPI_SWIGLU, true, g)) return e;
    g.A = Z, g.lda = d.F, g.W = w.wd, g.K = d.F, g.N = d.H, g.C = X, g.ldc = d.H;
    g.ssq_out = m->rSsq;
    if (int e = gemm_rows(m, EPI_RESID, false, g)) return e;
    nss = nss_h;
  }
  *nss_out = nss;
  return QDEC_OK;
}

// The decoder layers over T activation rows held in X (fp32 [T, H]), one
// layer after another (transcribe.cpp "Forward map - funasr_nano", table
// "LLM decoder"). rope(l) applies QK-norm + RoPE and appends K/V of layer l;
// attn(l, hi, lo) writes the attention output rows into Attn (fp32), or, when
// hi is set, as their bf16 hi/lo split into hi and lo (attn_split says whether
// it can); both return a status.
// With bf16 weights the attention writes the O projection's hi/lo operand
// itself, and on the tiled GEMM so does the SwiGLU GEMM for the down
// projection (the same bits the split pass would make); Z's fp32 buffer then
// holds Z hi and Z lo.
template <typename RopeFn, typename AttnFn>
int run_layers(qdec_model* m, int T, float* X, float* QKV, float* Attn, float* Z, void* A0, void* A1, RopeFn rope,
               AttnFn attn, bool attn_split) {
  const Dims& d = m->d;
  hipStream_t st = m->stream;
  const bool bf = m->bf16;
  auto norm_in = [&](const float* src, int K, const float* gain) -> hipError_t {
    if (bf) return launch_rms_split(src, T, K, gain, d.eps, (uint16_t*)A0, (uint16_t*)A1, st);
    return launch_rms_apply(src, T, K, gain, d.eps, (float*)A0, st);
  };
  const bool fuse_o = attn_split && bf;  // both bf16 GEMMs read the same hi/lo operand
  SplitK* sk = &m->split.sk;
  const bool fuse_z = gemm_tiled_fits(bf, T, d.H, 2 * d.F);  // the split epilogue is the tiled kernel's
  uint16_t* zhi = (uint16_t*)Z;
  uint16_t* zlo = zhi + (size_t)T * d.F;
  // a residual GEMM that splits K may apply the next RMSNorm in its
  // reduction (bf16 only: the fp32 path's operand is not split)
  auto resid_norm = [&](const float* gain) {
    return RowNorm{gain, d.eps, (uint16_t*)A0, (uint16_t*)A1, false};
  };
  bool in_done = false;
  for (int l = 0; l < d.L; ++l) {
    const LayerW& w = m->layers[l];
    if (!in_done) LAUNCH(norm_in(X, d.H, w.in_norm));
    LAUNCH(launch_gemm(bf, EPI_STORE, A0, A1, T, d.H, w.wqkv, d.qkv(), QKV, d.qkv(), st, nullptr, sk));
    if (int e = rope(l)) return e;
    if (fuse_o) {
      if (int e = attn(l, (uint16_t*)A0, (uint16_t*)A1)) return e;
    } else {
      if (int e = attn(l, nullptr, nullptr)) return e;
      LAUNCH(norm_in(Attn, d.NQ * d.D, nullptr));
    }
    RowNorm post = resid_norm(w.post_norm);
    LAUNCH(launch_gemm(bf, EPI_RESID, A0, A1, T, d.NQ * d.D, w.wo, d.H, X, d.H, st, nullptr, sk, bf ? &post : nullptr));
    if (!post.done) LAUNCH(norm_in(X, d.H, w.post_norm));
    RowNorm next = resid_norm(l + 1 < d.L ? m->layers[l + 1].in_norm : nullptr);
    RowNorm* nx = bf && l + 1 < d.L ? &next : nullptr;
    if (fuse_z) {
      LAUNCH(launch_gemm_swiglu_split((const uint16_t*)A0, (const uint16_t*)A1, T, d.H, (const uint16_t*)w.wgu,
                                      2 * d.F, zhi, zlo, d.F, st));
      LAUNCH(launch_gemm(bf, EPI_RESID, zhi, zlo, T, d.F, w.wd, d.H, X, d.H, st, nullptr, sk, nx));
    } else {
      LAUNCH(launch_gemm(bf, EPI_SWIGLU, A0, A1, T, d.H, w.wgu, 2 * d.F, Z, d.F, st, nullptr, sk));
      LAUNCH(norm_in(Z, d.F, nullptr));
      LAUNCH(launch_gemm(bf, EPI_RESID, A0, A1, T, d.F, w.wd, d.H, X, d.H, st, nullptr, sk, nx));
    }
    in_done = next.done;
  }
  return QDEC_OK;
}

// One decode step for n states at once: every weight is read once for all n
// rows; attention runs per row over that state's own pages.
int run_decode_batch(qdec_state* const* states, int n, const int32_t* tokens, float* logits, int32_t* argmax) {
  qdec_model* m = states[0]->m;
  const Dims& d = m->d;
  hipStream_t st = m->stream;
  BatchRows rows{};
  rows.n = n;
  int longest = 0;
  for (int i = 0; i < n; ++i) {
    rows.tok[i] = tokens[i];
    rows.pos[i] = states[i]->n_past;
    rows.pt[i] = states[i]->pt_dev;
    longest = std::max(longest, rows.pos[i] + 1);
  }
  const int nsplit = (longest + kAttnChunk - 1) / kAttnChunk;
  if (int e = ensure_batch(m, nsplit)) return e;
  if (__atomic_load_n(m->err_host, __ATOMIC_ACQUIRE))
    return fail(QDEC_E_DEVICE, "an earlier launch hit its time limit; the model must be recreated");
  const bool fused = use_rows(m, n);
  if (fused) {
    if (int e = ensure_rows(m)) return e;
  }
  float* lg = logits ? logits : m->bLogits;
  LAUNCH(launch_reset_keys(m->bKeys, n, st));
  LAUNCH(launch_embed_rows(d, m->bf16, m->embed, rows, m->bX, fused ? m->rSsq : nullptr, st));
  auto rope = [](int) { return 0; };  // inside the attention launch
  auto attn = [&](int l, uint16_t*, uint16_t*) -> int {  // fp32 output only
    const LayerW& w = m->layers[l];
    AttnRows a{};
    a.rows = rows;
    a.qkv = m->bQKV;
    a.layer = l;
    a.q_norm = w.q_norm;
    a.k_norm = w.k_norm;
    a.rcos = m->rope_cos;
    a.rsin = m->rope_sin;
    a.out = m->bAttn;
    a.part = m->bAttnPart;
    a.cnt = m->bAttnCnt;
    a.err = m->err_dev;
    if (int e = next_rows_tag(m, &a.tag)) return e;
    LAUNCH(launch_attn_rows(d, a, nsplit, st));
    return 0;
  };
  if (fused) {
    int nss = 1;
    if (int e = run_layers_rows(m, n, m->bX, m->bQKV, m->bAttn, m->bZ, 1, rope, attn, &nss)) return e;
    if (rows_fits(n, d.H, d.V)) {
      RowsGemm g{};
      g.A = m->bX, g.lda = d.H, g.ssq = m->rSsq, g.nss = nss, g.gain = m->final_norm, g.eps = d.eps;
      g.W = m->embed, g.M = n, g.K = d.H, g.N = d.V, g.P = m->rP, g.cnt = m->rCnt;
      g.C = logits, g.ldc = d.V, g.keys = m->bKeys;
      if (int e = gemm_rows(m, EPI_HEAD, true, g)) return e;
      LAUNCH(launch_argmax_final(m->bKeys, n, argmax ? argmax : m->bTok, st));
      return QDEC_OK;
    }
  } else if (int e = run_layers(m, n, m->bX, m->bQKV, m->bAttn, m->bZ, m->bA0, m->bA1, rope, attn, false)) {
    return e;
  }
  if (m->bf16)
    LAUNCH(launch_rms_split(m->bX, n, d.H, m->final_norm, d.eps, (uint16_t*)m->bA0, (uint16_t*)m->bA1, st));
  else
    LAUNCH(launch_rms_apply(m->bX, n, d.H, m->final_norm, d.eps, (float*)m->bA0, st));
  LAUNCH(launch_gemm(m->bf16, EPI_STORE, m->bA0, m->bA1, n, d.H, m->embed, d.V, lg, d.V, st));
  LAUNCH(launch_argmax_rows(lg, n, d.V, m->bKeys, st));
  LAUNCH(launch_argmax_final(m->bKeys, n, argmax ? argmax : m->bTok, st));
  return QDEC_OK;
}

int run_prefill(qdec_state* s, int T, const float* audio, int a0, int La, float* logits, int32_t* argmax) {
  qdec_model* m = s->m;
  const Dims& d = m->d;
  hipStream_t st = m->stream;
  const bool bf = m->bf16;
  // the fused path's workspace exists already (qdec_prefill allocates it
  // before anything is enqueued)
  const bool fused = use_rows(m, T);
  LAUNCH(launch_reset_keys(m->keys, 1, st));
  LAUNCH(launch_embed_prefill(d, bf, m->embed, m->p_ids, T, audio, a0, La, m->pX, fused ? m->rSsq : nullptr, st));
  // short prompts on the fused path: Q/K norm, RoPE, K/V append and the
  // attention in one launch per layer
  const bool small = fused && attn_small_fits(d, T);
  // the matrix-core attention applies the Q/K norm and RoPE and appends K/V
  // itself
  const bool fold = !small && attn_prefill_ropes(d);
  auto rope = [&](int l) -> int {
    if (small || fold) return 0;  // inside the attention launch
    const LayerW& w = m->layers[l];
    LAUNCH(launch_qk_rope_append(d, m->pQKV, T, 0, w.q_norm, w.k_norm, m->rope_cos, m->rope_sin, s->pt_dev, l, st));
    return 0;
  };
  auto attn = [&](int l, uint16_t* hi, uint16_t* lo) -> int {
    if (small) {
      const LayerW& w = m->layers[l];
      LAUNCH(launch_attn_small(d, m->pQKV, T, w.q_norm, w.k_norm, m->rope_cos, m->rope_sin, s->pt_dev, l, m->pAttn,
                               st));
      return 0;
    }
    const LayerW& w = m->layers[l];
    const QkRope rp{fold ? 1 : 0, w.q_norm, w.k_norm, m->rope_cos, m->rope_sin, s->pt_dev, l, d.L, 0, d.eps};
    LAUNCH(launch_attn_prefill(d, m->pQKV, T, m->pAttn, m->pKV, st, hi, lo, true, &m->split.sk, &rp));
    return 0;
  };
  if (fused) {
    int nss = 1;
    if (int e = run_layers_rows(m, T, m->pX, m->pQKV, m->pAttn, m->pZ, 1, rope, attn, &nss)) return e;
  } else if (int e = run_layers(m, T, m->pX, m->pQKV, m->pAttn, m->pZ, m->pA0, m->pA1, rope, attn,
                                attn_prefill_uses_split(d))) {
    return e;
  }
  LAUNCH(launch_lm_head(d, bf, m->embed, m->pX + (size_t)(T - 1) * d.H, m->final_norm, logits, m->keys, st));
  LAUNCH(launch_argmax_final(m->keys, 1, argmax ? argmax : m->argmax_tmp, st));
  return QDEC_OK;
}

int check_outputs(const qdec_model* m, int n, const float* logits, const int32_t* argmax) {
  if (logits) {
    if (int e = check_dev(logits, (size_t)n * m->d.V * sizeof(float), "logits_dev")) return e;
  }
  if (argmax) {
    if (int e = check_dev(argmax, (size_t)n * sizeof(int32_t), "argmax_dev")) return e;
  }
  return QDEC_OK;
}

int release_state_pages(qdec_state* s) {
  for (char* p : s->pages) s->m->pool.release(p);
  s->pages.clear();
  return QDEC_OK;
}

// Copies `bytes` from `src` to device `dst` on the model's stream through a
// pinned staging buffer, so the call returns without waiting for the copy.
// The buffer is reused only after its previous copy has completed.
int staged_upload(qdec_model* m, qdec_model::Staging& g, void* dst, const void* src, size_t bytes) {
  if (g.ev) HIP_TRY(hipEventSynchronize(g.ev));
  if (bytes > g.cap) {
    if (g.host) (void)hipHostFree(g.host);
    g.host = nullptr;
    g.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 4096);
    if (hipHostMalloc(&g.host, cap, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      g.host = nullptr;
      return fail(QDEC_E_OOM, "cannot allocate %zu bytes of pinned staging memory", cap);
    }
    g.cap = cap;
  }
  if (!g.ev) HIP_TRY(hipEventCreateWithFlags(&g.ev, hipEventDisableTiming));
  memcpy(g.host, src, bytes);
  HIP_TRY(hipMemcpyAsync(dst, g.host, bytes, hipMemcpyHostToDevice, m->stream));
  HIP_TRY(hipEventRecord(g.ev, m->stream));
  return QDEC_OK;
}

int upload_page_table(qdec_state* s) {
  std::vector<int64_t> pt(s->pages.size());
  for (size_t i = 0; i < pt.size(); ++i) pt[i] = (int64_t)(intptr_t)s->pages[i];
  return staged_upload(s->m, s->m->st_pt, s->pt_dev, pt.data(), pt.size() * sizeof(int64_t));
}

// The decode kernel's group-local exchange words (plain stores, non-temporal
// loads served by one XCD's L2) are correct only if every workgroup of group x
// (workgroups b with b % 8 == x) runs on one XCD. A probe launch of the decode
// kernel's shape records each workgroup's XCD; if some group spans two XCDs,
// or QDEC_EXCHANGE_SCOPE=device is set in the environment, those words use
// device scope instead (slower, placement-independent).
int check_placement(qdec_model* m) {
  m->dec_local = false;
  const char* env = getenv("QDEC_EXCHANGE_SCOPE");
  if (env && strcmp(env, "device") == 0) return QDEC_OK;
  const int nb = m->dec_blocks;
  int* d = nullptr;
  if (int e = dev_alloc(&d, (size_t)nb, "placement probe")) return e;
  std::vector<int> h(nb, -1);
  hipError_t he = launch_xcc_probe(m->wt, m->d, d, nb, m->dec_lds, m->stream);
  if (he == hipSuccess) he = hipMemcpyAsync(h.data(), d, nb * sizeof(int), hipMemcpyDeviceToHost, m->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(m->stream);
  (void)dfree(d);
  if (he != hipSuccess) return fail(QDEC_E_DEVICE, "placement probe: %s", hipGetErrorString(he));
  bool same = true;
  constexpr int kGroupCount = 8;  // decode groups (one per XCD)
  for (int b = kGroupCount; b < nb; ++b) same = same && h[b] == h[b % kGroupCount];
  m->dec_local = same;
  return QDEC_OK;
}

}  // namespace

// ================================================================= C ABI

extern "C" {

const char* qdec_last_error(void) { return g_err.c_str(); }

int qdec_create(const qdec_config* cfg, const qdec_weights* w, void* hip_stream, qdec_model** out) {
  if (!out) return fail(QDEC_E_INVALID, "out is NULL");
  *out = nullptr;
  if (int e = validate_config(cfg)) return e;
  if (!w || !w->embed || !w->final_norm || !w->layer) return fail(QDEC_E_INVALID, "weights incomplete");
  const qdec_config& c = *cfg;
  Dims d{c.n_layer, c.hidden, c.n_q_head, c.n_kv_head, c.head_dim, c.ffn, c.vocab, c.rms_eps};
  const bool q8 = c.weight_dtype == QDEC_Q8_0;
  // element size of every tensor (of the norm gains only, for Q8_0: fp32)
  const size_t es = c.weight_dtype == QDEC_BF16 ? 2 : 4;
  const size_t shp[QDEC_W_PER_LAYER] = {
      (size_t)d.H, (size_t)d.NQ * d.D * d.H, (size_t)d.NKV * d.D * d.H, (size_t)d.NKV * d.D * d.H,
      (size_t)d.D, (size_t)d.D, (size_t)d.H * d.NQ * d.D, (size_t)d.H, (size_t)d.F * d.H, (size_t)d.F * d.H,
      (size_t)d.H * d.F};
  const bool is_matrix[QDEC_W_PER_LAYER] = {false, true, true, true, false, false, true, false, true, true, true};
  // bytes of a matrix of n weights: Q8_0 blocks, or n elements
  auto mat_bytes = [&](size_t n) { return q8 ? n / kQ8Block * kQ8BlockBytes : n * es; };
  if (int e = check_dev(w->embed, mat_bytes((size_t)d.V * d.H), "embed")) return e;
  if (int e = check_dev(w->final_norm, (size_t)d.H * es, "final_norm")) return e;
  for (int l = 0; l < d.L; ++l)
    for (int t = 0; t < QDEC_W_PER_LAYER; ++t) {
      char what[64];
      snprintf(what, sizeof what, "layer %d tensor %d", l, t);
      const size_t nb = is_matrix[t] ? mat_bytes(shp[t]) : shp[t] * es;
      if (int e = check_dev(w->layer[l * QDEC_W_PER_LAYER + t], nb, what)) return e;
    }

  qdec_model* m = new (std::nothrow) qdec_model();
  if (!m) return fail(QDEC_E_OOM, "host allocation failed");
  m->cfg = c;
  m->d = d;
  m->bf16 = c.weight_dtype == QDEC_BF16;
  m->wt = c.weight_dtype;
  m->stream = (hipStream_t)hip_stream;
  m->embed = w->embed;
  m->pool.page_bytes = page_floats(d) * sizeof(float);
  hipStream_t st = m->stream;

  const size_t n_qkv = (size_t)d.qkv() * d.H, n_o = (size_t)d.H * d.NQ * d.D, n_gu = (size_t)2 * d.F * d.H,
               n_d = (size_t)d.H * d.F;
  const size_t per_layer = n_qkv + n_o + n_gu + n_d;
  const size_t norms_per_layer = 2 * (size_t)d.H + 2 * (size_t)d.D;
  int e = 0;
  if (dmalloc(&m->wbuf, per_layer * es * d.L) != hipSuccess) {
    (void)hipGetLastError();
    m->wbuf = nullptr;
    free_model(m);
    return fail(QDEC_E_OOM, "cannot allocate packed weights");
  }
  if ((e = dev_alloc(&m->nbuf, norms_per_layer * d.L, "norm gains")) ||
      (e = dev_alloc(&m->final_norm, d.H, "final norm")) || (e = dev_alloc(&m->keys, (size_t)kMaxBatch * kKeySlots, "argmax keys")) ||
      (e = dev_alloc(&m->argmax_tmp, kMaxBatch, "argmax scratch"))) {
    free_model(m);
    return e;
  }
  auto fail_dev = [&](const char* what, hipError_t he) {
    const int r = fail(QDEC_E_DEVICE, "%s: %s", what, hipGetErrorString(he));
    free_model(m);
    return r;
  };
  hipError_t he;
  char* wb = (char*)m->wbuf;
  m->layers.resize(d.L);
  if (q8) {
    // int8 codes in the packed row order, their segmented scales, and the
    // embedding as codes, scales and its exact fp32 dequantization
    const int QD = d.NQ / d.NKV * d.D, FS = d.F / 8;
    const size_t spH = q8_seg_bytes(d.H), spQD = q8_seg_bytes(QD), spFS = q8_seg_bytes(FS);
    m->soff_o = (size_t)d.qkv() * spH;
    m->soff_gu = m->soff_o + (size_t)d.H * d.NKV * spQD;
    m->soff_d = m->soff_gu + (size_t)2 * d.F * spH;
    m->layer_sbytes = m->soff_d + (size_t)d.H * 8 * spFS;
    const size_t sbytes = m->layer_sbytes * d.L + kQ8ScalePad, esbytes = (size_t)d.V * spH + kQ8ScalePad;
    if ((e = dev_alloc(&m->q_codes, per_layer * d.L, "int8 weight codes")) ||
        (e = dev_alloc(&m->q_scales, sbytes / 2, "weight scales")) ||
        (e = dev_alloc(&m->q_embed, (size_t)d.V * d.H, "int8 embedding codes")) ||
        (e = dev_alloc(&m->q_escale, esbytes / 2, "embedding scales")) ||
        (e = dev_alloc(&m->embed_own, (size_t)d.V * d.H, "dequantized embedding"))) {
      free_model(m);
      return e;
    }
    m->embed = m->embed_own;
    // padding between and after segments reads as zero scales
    if ((he = hipMemsetAsync(m->q_scales, 0, sbytes, st)) || (he = hipMemsetAsync(m->q_escale, 0, esbytes, st)))
      return fail_dev("scale init", he);
    if ((he = launch_q8_unpack(w->embed, d.V, d.H, d.H, 0, -1, m->q_embed, m->q_escale, m->embed_own, st)))
      return fail_dev("unpack embed", he);
  }
  for (int l = 0; l < d.L; ++l) {
    const void* const* t = w->layer + (size_t)l * QDEC_W_PER_LAYER;
    char* base = wb + per_layer * es * l;
    char* qkv = base;
    char* o = qkv + n_qkv * es;
    char* gu = o + n_o * es;
    char* dn = gu + n_gu * es;
    float* nb = m->nbuf + norms_per_layer * l;
    if (q8) {
      int8_t* cb = m->q_codes + per_layer * l;
      uint16_t* sb = m->q_scales + m->layer_sbytes * l / 2;
      float* fb = (float*)base;
      const int QD = d.NQ / d.NKV * d.D;
      struct Part {
        int t, rows, K, kseg, row0, gu_half;
        size_t off, soff;
      };
      const Part parts[] = {{QDEC_W_Q, d.NQ * d.D, d.H, d.H, 0, -1, 0, 0},
                            {QDEC_W_K, d.NKV * d.D, d.H, d.H, d.NQ * d.D, -1, 0, 0},
                            {QDEC_W_V, d.NKV * d.D, d.H, d.H, (d.NQ + d.NKV) * d.D, -1, 0, 0},
                            {QDEC_W_O, d.H, d.NQ * d.D, QD, 0, -1, n_qkv, m->soff_o},
                            {QDEC_W_GATE, d.F, d.H, d.H, 0, 0, n_qkv + n_o, m->soff_gu},
                            {QDEC_W_UP, d.F, d.H, d.H, 0, 1, n_qkv + n_o, m->soff_gu},
                            {QDEC_W_DOWN, d.H, d.F, d.F / 8, 0, -1, n_qkv + n_o + n_gu, m->soff_d}};
      for (const Part& pt : parts)
        if ((he = launch_q8_unpack(t[pt.t], pt.rows, pt.K, pt.kseg, pt.row0, pt.gu_half, cb + pt.off,
                                   sb + pt.soff / 2, fb + pt.off, st)))
          return fail_dev("unpack weights", he);
    } else {
      const size_t row = (size_t)d.H * es;
      size_t off = 0;
      if ((he = hipMemcpyAsync(qkv + off, t[QDEC_W_Q], shp[QDEC_W_Q] * es, hipMemcpyDeviceToDevice, st)))
        return fail_dev("pack wq", he);
      off += shp[QDEC_W_Q] * es;
      if ((he = hipMemcpyAsync(qkv + off, t[QDEC_W_K], shp[QDEC_W_K] * es, hipMemcpyDeviceToDevice, st)))
        return fail_dev("pack wk", he);
      off += shp[QDEC_W_K] * es;
      if ((he = hipMemcpyAsync(qkv + off, t[QDEC_W_V], shp[QDEC_W_V] * es, hipMemcpyDeviceToDevice, st)))
        return fail_dev("pack wv", he);
      if ((he = hipMemcpyAsync(o, t[QDEC_W_O], n_o * es, hipMemcpyDeviceToDevice, st))) return fail_dev("pack wo", he);
      // gate/up interleaved in groups of kGuGroup rows
      const size_t grp = (size_t)kGuGroup * row;
      if ((he = hipMemcpy2DAsync(gu, 2 * grp, t[QDEC_W_GATE], grp, grp, d.F / kGuGroup, hipMemcpyDeviceToDevice, st)))
        return fail_dev("pack gate", he);
      if ((he = hipMemcpy2DAsync(gu + grp, 2 * grp, t[QDEC_W_UP], grp, grp, d.F / kGuGroup, hipMemcpyDeviceToDevice,
                                 st)))
        return fail_dev("pack up", he);
      if ((he = hipMemcpyAsync(dn, t[QDEC_W_DOWN], n_d * es, hipMemcpyDeviceToDevice, st)))
        return fail_dev("pack down", he);
    }
    if ((he = launch_to_f32(t[QDEC_W_IN_NORM], m->bf16, d.H, nb, st))) return fail_dev("in_norm", he);
    if ((he = launch_to_f32(t[QDEC_W_POST_NORM], m->bf16, d.H, nb + d.H, st))) return fail_dev("post_norm", he);
    if ((he = launch_to_f32(t[QDEC_W_Q_NORM], m->bf16, d.D, nb + 2 * d.H, st))) return fail_dev("q_norm", he);
    if ((he = launch_to_f32(t[QDEC_W_K_NORM], m->bf16, d.D, nb + 2 * d.H + d.D, st))) return fail_dev("k_norm", he);
    m->layers[l] = LayerW{qkv, o, gu, dn, nb, nb + d.H, nb + 2 * d.H, nb + 2 * d.H + d.D};
  }
  if ((he = launch_to_f32(w->final_norm, m->bf16, d.H, m->final_norm, st))) return fail_dev("final_norm", he);
  m->layer_elems = per_layer;
  m->off_o = n_qkv;
  m->off_gu = n_qkv + n_o;
  m->off_d = n_qkv + n_o + n_gu;
  m->norm_elems = (int)norms_per_layer;
  // persistent decode: one workgroup per CU, all resident at once (one per CU by LDS)
  {
    int dev = 0;
    hipDeviceProp_t prop;
    if ((he = hipGetDevice(&dev)) || (he = hipGetDeviceProperties(&prop, dev))) return fail_dev("device query", he);
    m->dec_blocks = prop.multiProcessorCount;
    if (m->dec_blocks < 8 || m->dec_blocks % 8) {
      free_model(m);
      return fail(QDEC_E_INVALID, "decode needs a multiple of 8 compute units (device has %d)", m->dec_blocks);
    }
    if (!dec_fits(m->wt, d, m->dec_blocks)) {
      free_model(m);
      return fail(QDEC_E_INVALID, "shape too large for the decode kernel's LDS staging on %d CUs", m->dec_blocks);
    }
    m->nsplit_max = dec_split_limit(d, m->dec_blocks);
    m->whole_max = 64;
    // dynamic LDS; the kernel's static weight rings (96 KB) already keep the
    // runtime from placing two workgroups on one CU
    m->dec_lds = dec_lds_bytes(m->wt, d, m->dec_blocks, m->nsplit_max);
    int occ = 0;
    if ((he = dec_prepare(m->wt, d, m->dec_lds, &occ))) return fail_dev("decode kernel setup", he);
    if (occ != 1) {
      free_model(m);
      return fail(QDEC_E_INVALID, "decode kernel must fit exactly one workgroup per CU (got %d, LDS %zu bytes)", occ,
                  m->dec_lds);
    }
    m->ll_words = dec_words(d, m->dec_blocks, m->nsplit_max, &m->off);
    if ((e = dev_alloc(&m->ll, m->ll_words, "exchange words"))) {
      free_model(m);
      return e;
    }
    if ((he = launch_clear_words(m->ll, m->ll_words, st))) return fail_dev("exchange init", he);
    if ((e = check_placement(m))) {
      free_model(m);
      return e;
    }
    // the fixed sampling scratch of this device (qdec_sample_noalloc)
    if ((he = sample_static_scratch(&m->sStatic0, &m->sStatic1))) return fail_dev("sampling scratch address", he);
    if ((he = hipHostMalloc((void**)&m->err_host, sizeof(int), hipHostMallocMapped))) {
      m->err_host = nullptr;
      return fail_dev("error flag", he);
    }
    *m->err_host = 0;
    if ((he = hipHostGetDevicePointer((void**)&m->err_dev, m->err_host, 0))) return fail_dev("error flag map", he);
    if ((e = alloc_splitk(&m->split))) {
      free_model(m);
      return e;
    }
  }
  if ((he = hipStreamSynchronize(st))) return fail_dev("weight packing", he);
  if ((e = ensure_rope(m, 4096))) {
    free_model(m);
    return e;
  }
  *out = m;
  return ok();
}

int qdec_destroy(qdec_model* m) {
  if (!m) return ok();
  if (m->live_states > 0) return fail(QDEC_E_STATE, "%d states of this model are still alive", m->live_states);
  free_model(m);
  return ok();
}

int qdec_state_create(qdec_model* m, int32_t max_ctx, qdec_state** out) {
  if (!out) return fail(QDEC_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!m) return fail(QDEC_E_INVALID, "model is NULL");
  if (max_ctx < 1 || max_ctx > (1 << 20)) return fail(QDEC_E_INVALID, "max_ctx %d out of range", max_ctx);
  if (int e = ensure_rope(m, max_ctx)) return e;
  const int npages = (max_ctx + kPage - 1) / kPage;
  if (int e = m->pool.reserve(npages)) return e;
  qdec_state* s = new (std::nothrow) qdec_state();
  if (!s) return fail(QDEC_E_OOM, "host allocation failed");
  s->m = m;
  s->max_ctx = max_ctx;
  if (int e = dev_alloc(&s->pt_dev, npages, "page table")) {
    delete s;
    return e;
  }
  for (int i = 0; i < npages; ++i) s->pages.push_back(m->pool.take());
  if (int e = upload_page_table(s)) {
    release_state_pages(s);
    (void)dfree(s->pt_dev);
    delete s;
    return e;
  }
  ++m->live_states;
  *out = s;
  return ok();
}

void qdec_state_destroy(qdec_state* s) {
  if (!s) return;
  (void)hipStreamSynchronize(s->m->stream);
  release_state_pages(s);
  (void)dfree(s->pt_dev);
  --s->m->live_states;
  delete s;
}

int32_t qdec_state_pos(const qdec_state* s) { return s ? s->n_past : -1; }

int qdec_model_status(const qdec_model* m) {
  if (!m) return fail(QDEC_E_INVALID, "model is NULL");
  if (__atomic_load_n(m->err_host, __ATOMIC_ACQUIRE))
    return fail(QDEC_E_DEVICE, "a device-side wait hit its time limit; outputs since then are invalid");
  return ok();
}

int qdec_prefill(qdec_state* s, const int32_t* ids_host, int32_t n_tokens, const float* audio_dev,
                 int32_t audio_begin, int32_t audio_len, float* logits_dev, int32_t* argmax_dev) {
  if (!s) return fail(QDEC_E_INVALID, "state is NULL");
  qdec_model* m = s->m;
  if (s->n_past != 0) return fail(QDEC_E_STATE, "prefill needs an empty state (n_past = %d)", s->n_past);
  if (n_tokens < 1) return fail(QDEC_E_INVALID, "n_tokens %d < 1", n_tokens);
  if (n_tokens > s->max_ctx)
    return fail(QDEC_E_CAPACITY, "n_tokens %d exceeds max_ctx %d", n_tokens, s->max_ctx);
  if (!ids_host) return fail(QDEC_E_INVALID, "ids_host is NULL");
  if (audio_begin < 0 || audio_len < 0 || (int64_t)audio_begin + audio_len > n_tokens)
    return fail(QDEC_E_INVALID, "audio span [%d, %d + %d) outside the prompt of %d", audio_begin, audio_begin,
                audio_len, n_tokens);
  if (audio_len > 0) {
    if (int e = check_dev(audio_dev, (size_t)audio_len * m->d.H * sizeof(float), "audio_dev")) return e;
  }
  for (int t = 0; t < n_tokens; ++t) {
    if (t >= audio_begin && t < audio_begin + audio_len) continue;
    if (ids_host[t] < 0 || ids_host[t] >= m->d.V)
      return fail(QDEC_E_INVALID, "ids[%d] = %d outside [0, %d)", t, ids_host[t], m->d.V);
  }
  if (int e = check_outputs(m, 1, logits_dev, argmax_dev)) return e;
  if (__atomic_load_n(m->err_host, __ATOMIC_ACQUIRE))
    return fail(QDEC_E_DEVICE, "an earlier launch hit its time limit; the model must be recreated");
  if (int e = ensure_prefill(m, n_tokens)) return e;
  if (use_rows(m, n_tokens)) {
    if (int e = ensure_rows(m)) return e;
  }
  std::vector<int32_t> ids(ids_host, ids_host + n_tokens);
  for (int t = audio_begin; t < audio_begin + audio_len; ++t) ids[t] = 0;  // never read
  if (int e = staged_upload(m, m->st_ids, m->p_ids, ids.data(), n_tokens * sizeof(int32_t))) return e;
  if (int e = run_prefill(s, n_tokens, audio_dev, audio_begin, audio_len, logits_dev, argmax_dev)) return e;
  s->n_past = n_tokens;
  return ok();
}

static int decode_common(qdec_state* s, int token, const int32_t* token_dev, int32_t pos, float* logits_dev,
                         int32_t* argmax_dev) {
  if (!s) return fail(QDEC_E_INVALID, "state is NULL");
  if (pos != s->n_past) return fail(QDEC_E_POS, "pos %d != n_past %d", pos, s->n_past);
  if (pos >= s->max_ctx) return fail(QDEC_E_CAPACITY, "pos %d >= max_ctx %d", pos, s->max_ctx);
  if (int e = check_outputs(s->m, 1, logits_dev, argmax_dev)) return e;
  if (int e = run_decode(s, token, token_dev, pos, 1, logits_dev, argmax_dev)) return e;
  s->n_past = pos + 1;
  return ok();
}

int qdec_decode_step(qdec_state* s, int32_t token, int32_t pos, float* logits_dev, int32_t* argmax_dev) {
  if (s && (token < 0 || token >= s->m->d.V))
    return fail(QDEC_E_INVALID, "token %d outside [0, %d)", token, s->m->d.V);
  return decode_common(s, token, nullptr, pos, logits_dev, argmax_dev);
}

int qdec_decode_step_dev(qdec_state* s, const int32_t* token_dev, int32_t pos, float* logits_dev,
                         int32_t* argmax_dev) {
  if (int e = check_dev(token_dev, sizeof(int32_t), "token_dev")) return e;
  return decode_common(s, 0, token_dev, pos, logits_dev, argmax_dev);
}

int qdec_decode_greedy(qdec_state* s, const int32_t* token_dev, int32_t pos, int32_t n_steps, float* logits_dev,
                       int32_t* tokens_dev) {
  if (!s) return fail(QDEC_E_INVALID, "state is NULL");
  if (n_steps < 1 || n_steps > 4096) return fail(QDEC_E_INVALID, "n_steps %d outside [1, 4096]", n_steps);
  if (pos != s->n_past) return fail(QDEC_E_POS, "pos %d != n_past %d", pos, s->n_past);
  if ((int64_t)pos + n_steps > s->max_ctx)
    return fail(QDEC_E_CAPACITY, "pos %d + n_steps %d exceeds max_ctx %d", pos, n_steps, s->max_ctx);
  if (int e = check_dev(token_dev, sizeof(int32_t), "token_dev")) return e;
  if (int e = check_dev(tokens_dev, (size_t)n_steps * sizeof(int32_t), "tokens_dev")) return e;
  if (logits_dev) {
    if (int e = check_dev(logits_dev, (size_t)n_steps * s->m->d.V * sizeof(float), "logits_dev")) return e;
  }
  if (int e = run_decode(s, 0, token_dev, pos, n_steps, logits_dev, tokens_dev)) return e;
  s->n_past = pos + n_steps;
  return ok();
}

int qdec_decode_batch(qdec_state* const* states, int32_t n, const int32_t* tokens_host, float* logits_dev,
                      int32_t* argmax_dev) {
  if (!states || !tokens_host) return fail(QDEC_E_INVALID, "states or tokens_host is NULL");
  if (n < 1 || n > kMaxBatch) return fail(QDEC_E_INVALID, "batch %d outside [1, %d]", n, kMaxBatch);
  qdec_model* m = states[0] ? states[0]->m : nullptr;
  if (!m) return fail(QDEC_E_INVALID, "states[0] is NULL");
  for (int i = 0; i < n; ++i) {
    qdec_state* s = states[i];
    if (!s || s->m != m) return fail(QDEC_E_INVALID, "states[%d] is NULL or of another model", i);
    for (int j = 0; j < i; ++j)
      if (states[j] == s) return fail(QDEC_E_INVALID, "states[%d] repeats states[%d]", i, j);
    if (s->n_past >= s->max_ctx)
      return fail(QDEC_E_CAPACITY, "states[%d]: n_past %d == max_ctx", i, s->n_past);
    if (tokens_host[i] < 0 || tokens_host[i] >= m->d.V)
      return fail(QDEC_E_INVALID, "tokens[%d] = %d outside [0, %d)", i, tokens_host[i], m->d.V);
  }
  if (int e = check_outputs(m, n, logits_dev, argmax_dev)) return e;
  if (int e = run_decode_batch(states, n, tokens_host, logits_dev, argmax_dev)) return e;
  for (int i = 0; i < n; ++i) states[i]->n_past += 1;
  return ok();
}

}  // extern "C"

namespace {

// Checks the arguments of a sampling call (both entry points) and fills u.
int sample_args(qdec_model* m, const float* logits_dev, int32_t n_rows, const qdec_sampling* params,
                const int32_t* history_dev, int32_t history_len, const float* uniforms_host, int32_t* tokens_dev,
                SampleUniforms* u) {
  if (!m || !params || !uniforms_host) return fail(QDEC_E_INVALID, "model, params or uniforms_host is NULL");
  const Dims& d = m->d;
  if (n_rows < 1 || n_rows > kMaxBatch) return fail(QDEC_E_INVALID, "n_rows %d outside [1, %d]", n_rows, kMaxBatch);
  const qdec_sampling& p = *params;
  if (!(p.temperature >= 0.f) || !std::isfinite(p.temperature))
    return fail(QDEC_E_INVALID, "temperature must be finite and >= 0");
  if (p.temperature > 0.f && (p.top_k < 1 || p.top_k > QDEC_SAMPLE_TOP_K_MAX || p.top_k > d.V))
    return fail(QDEC_E_INVALID, "top_k %d outside [1, %d]", p.top_k, std::min(QDEC_SAMPLE_TOP_K_MAX, d.V));
  if (!(p.top_p > 0.f && p.top_p <= 1.f)) return fail(QDEC_E_INVALID, "top_p must lie in (0, 1]");
  if (!(p.repetition_penalty > 0.f) || !std::isfinite(p.repetition_penalty))
    return fail(QDEC_E_INVALID, "repetition_penalty must be finite and > 0");
  if (history_len < 0 || (history_len > 0 && !history_dev))
    return fail(QDEC_E_INVALID, "history_len %d with history_dev %p", history_len, (const void*)history_dev);
  for (int r = 0; r < n_rows; ++r) {
    if (!(uniforms_host[r] >= 0.f && uniforms_host[r] < 1.f))
      return fail(QDEC_E_INVALID, "uniforms_host[%d] outside [0, 1)", r);
    u->u[r] = uniforms_host[r];
  }
  if (int e = check_dev(logits_dev, (size_t)n_rows * d.V * sizeof(float), "logits_dev")) return e;
  if (int e = check_dev(tokens_dev, (size_t)n_rows * sizeof(int32_t), "tokens_dev")) return e;
  if (history_len > 0) {
    if (int e = check_dev(history_dev, (size_t)n_rows * history_len * sizeof(int32_t), "history_dev")) return e;
  }
  return QDEC_OK;
}

}  // namespace

extern "C" {

int qdec_sample(qdec_model* m, const float* logits_dev, int32_t n_rows, const qdec_sampling* params,
                const int32_t* history_dev, int32_t history_len, const float* uniforms_host, int32_t* tokens_dev) {
  SampleUniforms u{};
  if (int e = sample_args(m, logits_dev, n_rows, params, history_dev, history_len, uniforms_host, tokens_dev, &u))
    return e;
  const Dims& d = m->d;
  const qdec_sampling& p = *params;
  if (!m->sBuf0) {
    const size_t words = sample_buffer_words(d.V);
    if (int e = dev_alloc(&m->sBuf0, words, "sampling buffer")) return e;
    if (int e = dev_alloc(&m->sBuf1, words, "sampling buffer")) {
      (void)dfree(m->sBuf0);
      m->sBuf0 = nullptr;
      return e;
    }
  }
  LAUNCH(launch_sample(logits_dev, n_rows, d.V, history_dev, history_len, p.repetition_penalty, p.temperature,
                       p.top_k, p.top_p, u, m->sBuf0, m->sBuf1, tokens_dev, m->stream));
  return ok();
}

int qdec_sample_noalloc(qdec_model* m, const float* logits_dev, int32_t n_rows, const qdec_sampling* params,
                        const int32_t* history_dev, int32_t history_len, const float* uniforms_host,
                        int32_t* tokens_dev) {
  SampleUniforms u{};
  if (int e = sample_args(m, logits_dev, n_rows, params, history_dev, history_len, uniforms_host, tokens_dev, &u))
    return e;
  const Dims& d = m->d;
  if (d.V > sample_static_max_vocab())
    return fail(QDEC_E_INVALID, "vocab %d exceeds the %d entries the fixed sampling scratch holds", d.V,
                sample_static_max_vocab());
  const qdec_sampling& p = *params;
  // the device's fixed scratch (address resolved at qdec_create); every
  // buffer word a level reads was written by the level before it, so nothing
  // needs clearing
  LAUNCH(launch_sample(logits_dev, n_rows, d.V, history_dev, history_len, p.repetition_penalty, p.temperature,
                       p.top_k, p.top_p, u, m->sStatic0, m->sStatic1, tokens_dev, m->stream));
  return ok();
}

int qdec_clone_state(const qdec_state* src, qdec_state** dst) {
  if (!dst) return fail(QDEC_E_INVALID, "dst is NULL");
  *dst = nullptr;
  if (!src) return fail(QDEC_E_INVALID, "src is NULL");
  qdec_model* m = src->m;
  const int npages = (int)src->pages.size();
  const int nfull = src->n_past / kPage;
  const bool tail = src->n_past % kPage != 0;
  if (int e = m->pool.reserve(npages - nfull)) return e;
  qdec_state* s = new (std::nothrow) qdec_state();
  if (!s) return fail(QDEC_E_OOM, "host allocation failed");
  s->m = m;
  s->max_ctx = src->max_ctx;
  s->n_past = src->n_past;
  if (int e = dev_alloc(&s->pt_dev, npages, "page table")) {
    delete s;
    return e;
  }
  for (int i = 0; i < nfull; ++i) {
    m->pool.retain(src->pages[i]);
    s->pages.push_back(src->pages[i]);
  }
  for (int i = nfull; i < npages; ++i) s->pages.push_back(m->pool.take());
  if (tail) {
    if (hipMemcpyAsync(s->pages[nfull], src->pages[nfull], m->pool.page_bytes, hipMemcpyDeviceToDevice, m->stream) !=
        hipSuccess) {
      (void)hipGetLastError();
      release_state_pages(s);
      (void)dfree(s->pt_dev);
      delete s;
      return fail(QDEC_E_DEVICE, "tail page copy failed");
    }
  }
  if (int e = upload_page_table(s)) {
    release_state_pages(s);
    (void)dfree(s->pt_dev);
    delete s;
    return e;
  }
  ++m->live_states;
  *dst = s;
  return ok();
}

}  // extern "C"

// ================================================================= adaptor
// The audio adaptor (transcribe.cpp "Forward map - funasr_nano", section
// "Adaptor"): linear1 + ReLU, linear2, then pre-norm blocks of biased MHA with
// every frame attending to every frame, and a ReLU FFN. All on the prefill
// kernels: bf16 hi/lo split operands, the tiled (or small-M) MFMA GEMMs with
// bias / ReLU / residual epilogues, LayerNorm written as the next GEMM's
// operand, and the matrix-core attention without the causal mask.

struct qdec_adaptor {
  qdec_adaptor_config c{};
  hipStream_t stream = nullptr;
  const uint16_t* w1 = nullptr;
  const uint16_t* w2 = nullptr;
  float* b1 = nullptr;
  float* b2 = nullptr;
  struct Block {
    uint16_t* wqkv = nullptr;  // [3 dim, dim]: q rows, k rows, v rows
    const uint16_t *wo = nullptr, *fc1 = nullptr, *fc2 = nullptr;
    float *bqkv = nullptr, *bo = nullptr, *n1g = nullptr, *n1b = nullptr, *n2g = nullptr, *n2b = nullptr;
    float *bf1 = nullptr, *bf2 = nullptr;
  };
  std::vector<Block> blocks;
  float* vecs = nullptr;  // every bias and norm vector, fp32
  SplitKBuf split;        // split-K workspace of the GEMMs
  // scratch for up to `cap` frames
  int cap = 0;
  uint16_t* A0 = nullptr;  // bf16 hi of the current GEMM operand
  uint16_t* A1 = nullptr;  // bf16 lo
  float* H = nullptr;      // linear1 / fc1 output
  float* QKV = nullptr;
  uint16_t* kv[4] = {nullptr, nullptr, nullptr, nullptr};
};

namespace {

Dims adaptor_dims(const qdec_adaptor_config& c) {
  return Dims{1, c.dim, c.n_head, c.n_head, c.dim / c.n_head, 0, 0, 0.f};
}

void free_adaptor_scratch(qdec_adaptor* a) {
  for (void* p : {(void*)a->A0, (void*)a->A1, (void*)a->H, (void*)a->QKV, (void*)a->kv[0], (void*)a->kv[1],
                  (void*)a->kv[2], (void*)a->kv[3]})
    if (p) (void)dfree(p);
  a->A0 = a->A1 = nullptr;
  a->H = a->QKV = nullptr;
  for (auto& k : a->kv) k = nullptr;
  a->cap = 0;
}

void free_adaptor(qdec_adaptor* a) {
  if (!a) return;
  (void)hipStreamSynchronize(a->stream);
  free_adaptor_scratch(a);
  for (auto& b : a->blocks)
    if (b.wqkv) (void)dfree(b.wqkv);
  if (a->vecs) (void)dfree(a->vecs);
  free_splitk(&a->split);
  delete a;
}

int ensure_adaptor(qdec_adaptor* a, int T) {
  if (T <= a->cap) return QDEC_OK;
  free_adaptor_scratch(a);
  const qdec_adaptor_config& c = a->c;
  const size_t wide = (size_t)std::max(std::max(c.enc_dim, c.mid_dim), std::max(c.dim, c.ffn_dim));
  const size_t Tp = (size_t)kv_split_pad(T);
  int e;
  if ((e = dev_alloc(&a->A0, (size_t)T * wide, "adaptor operand")) ||
      (e = dev_alloc(&a->A1, (size_t)T * wide, "adaptor operand")) ||
      (e = dev_alloc(&a->H, (size_t)T * std::max(c.mid_dim, c.ffn_dim), "adaptor hidden")) ||
      (e = dev_alloc(&a->QKV, (size_t)T * 3 * c.dim, "adaptor qkv")) ||
      (e = dev_alloc(&a->kv[0], (size_t)T * c.dim, "adaptor K")) ||
      (e = dev_alloc(&a->kv[1], (size_t)T * c.dim, "adaptor K")) ||
      (e = dev_alloc(&a->kv[2], Tp * c.dim, "adaptor V")) || (e = dev_alloc(&a->kv[3], Tp * c.dim, "adaptor V"))) {
    free_adaptor_scratch(a);
    return e;
  }
  a->cap = T;
  return QDEC_OK;
}

}  // namespace

extern "C" {

int qdec_adaptor_create(const qdec_adaptor_config* cfg, const qdec_adaptor_weights* w, void* hip_stream,
                        qdec_adaptor** out) {
  if (!out) return fail(QDEC_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(QDEC_E_INVALID, "config is NULL");
  const qdec_adaptor_config& c = *cfg;
  if (c.weight_dtype != QDEC_BF16) return fail(QDEC_E_INVALID, "the adaptor takes bf16 weights");
  if (c.enc_dim < 32 || c.enc_dim % 32 || c.mid_dim < 128 || c.mid_dim % 128 || c.ffn_dim < 128 ||
      c.ffn_dim % 128)
    return fail(QDEC_E_INVALID, "enc_dim %d (multiple of 32), mid_dim %d and ffn_dim %d (multiples of 128)",
                c.enc_dim, c.mid_dim, c.ffn_dim);
  if (c.n_head < 1 || c.n_head > 64 || c.dim != c.n_head * 128)
    return fail(QDEC_E_INVALID, "dim %d must be n_head (%d) * 128", c.dim, c.n_head);
  if (c.n_block < 1 || c.n_block > 8) return fail(QDEC_E_INVALID, "n_block %d outside 1 .. 8", c.n_block);
  if (!(c.ln_eps > 0.f) || !std::isfinite(c.ln_eps)) return fail(QDEC_E_INVALID, "ln_eps must be > 0");
  if (!w || !w->linear1_w || !w->linear1_b || !w->linear2_w || !w->linear2_b || !w->block)
    return fail(QDEC_E_INVALID, "adaptor weights incomplete");
  const size_t D = c.dim, F = c.ffn_dim;
  if (int e = check_dev(w->linear1_w, (size_t)c.mid_dim * c.enc_dim * 2, "linear1_w")) return e;
  if (int e = check_dev(w->linear1_b, (size_t)c.mid_dim * 2, "linear1_b")) return e;
  if (int e = check_dev(w->linear2_w, D * c.mid_dim * 2, "linear2_w")) return e;
  if (int e = check_dev(w->linear2_b, D * 2, "linear2_b")) return e;
  for (int b = 0; b < c.n_block; ++b) {
    const void* const* t = w->block + (size_t)b * QDEC_AB_PER_BLOCK;
    for (int i = 0; i < QDEC_AB_PER_BLOCK; ++i) {
      const bool mat = i == QDEC_AB_Q_W || i == QDEC_AB_K_W || i == QDEC_AB_V_W || i == QDEC_AB_O_W ||
                       i == QDEC_AB_FC1_W || i == QDEC_AB_FC2_W;
      const size_t n = i == QDEC_AB_FC1_W || i == QDEC_AB_FC2_W ? F * D : mat ? D * D : i == QDEC_AB_FC1_B ? F : D;
      char what[48];
      snprintf(what, sizeof what, "block %d tensor %d", b, i);
      if (int e = check_dev(t[i], n * 2, what)) return e;
    }
  }
  qdec_adaptor* a = new (std::nothrow) qdec_adaptor();
  if (!a) return fail(QDEC_E_OOM, "host allocation failed");
  a->c = c;
  a->stream = (hipStream_t)hip_stream;
  a->w1 = (const uint16_t*)w->linear1_w;
  a->w2 = (const uint16_t*)w->linear2_w;
  const size_t per_block = 9 * D + F;
  const size_t nvec = (size_t)c.mid_dim + D + (size_t)c.n_block * per_block;
  if (int e = dev_alloc(&a->vecs, nvec, "adaptor vectors")) {
    free_adaptor(a);
    return e;
  }
  hipStream_t st = a->stream;
  if (int e = alloc_splitk(&a->split)) {
    free_adaptor(a);
    return e;
  }
  auto fail_dev = [&](const char* what, hipError_t he) {
    const int r = fail(QDEC_E_DEVICE, "%s: %s", what, hipGetErrorString(he));
    free_adaptor(a);
    return r;
  };
  hipError_t he;
  float* v = a->vecs;
  a->b1 = v;
  v += c.mid_dim;
  a->b2 = v;
  v += D;
  if ((he = launch_to_f32(w->linear1_b, true, c.mid_dim, a->b1, st))) return fail_dev("linear1_b", he);
  if ((he = launch_to_f32(w->linear2_b, true, D, a->b2, st))) return fail_dev("linear2_b", he);
  a->blocks.resize(c.n_block);
  for (int b = 0; b < c.n_block; ++b) {
    const void* const* t = w->block + (size_t)b * QDEC_AB_PER_BLOCK;
    qdec_adaptor::Block& k = a->blocks[b];
    if (int e = dev_alloc(&k.wqkv, 3 * D * D, "adaptor wqkv")) {
      free_adaptor(a);
      return e;
    }
    const size_t mb = D * D * 2;
    if ((he = hipMemcpyAsync(k.wqkv, t[QDEC_AB_Q_W], mb, hipMemcpyDeviceToDevice, st)) ||
        (he = hipMemcpyAsync(k.wqkv + D * D, t[QDEC_AB_K_W], mb, hipMemcpyDeviceToDevice, st)) ||
        (he = hipMemcpyAsync(k.wqkv + 2 * D * D, t[QDEC_AB_V_W], mb, hipMemcpyDeviceToDevice, st)))
      return fail_dev("pack wqkv", he);
    k.wo = (const uint16_t*)t[QDEC_AB_O_W];
    k.fc1 = (const uint16_t*)t[QDEC_AB_FC1_W];
    k.fc2 = (const uint16_t*)t[QDEC_AB_FC2_W];
    k.bqkv = v;
    k.bo = v + 3 * D;
    k.n1g = v + 4 * D;
    k.n1b = v + 5 * D;
    k.n2g = v + 6 * D;
    k.n2b = v + 7 * D;
    k.bf2 = v + 8 * D;
    k.bf1 = v + 9 * D;
    v += per_block;
    const struct {
      int idx;
      float* dst;
      size_t n;
    } vecs[] = {{QDEC_AB_Q_B, k.bqkv, D}, {QDEC_AB_K_B, k.bqkv + D, D}, {QDEC_AB_V_B, k.bqkv + 2 * D, D},
                {QDEC_AB_O_B, k.bo, D},   {QDEC_AB_NORM1_G, k.n1g, D},  {QDEC_AB_NORM1_B, k.n1b, D},
                {QDEC_AB_NORM2_G, k.n2g, D}, {QDEC_AB_NORM2_B, k.n2b, D}, {QDEC_AB_FC2_B, k.bf2, D},
                {QDEC_AB_FC1_B, k.bf1, F}};
    for (const auto& x : vecs)
      if ((he = launch_to_f32(t[x.idx], true, x.n, x.dst, st))) return fail_dev("adaptor vector", he);
  }
  if ((he = hipStreamSynchronize(st))) return fail_dev("adaptor packing", he);
  *out = a;
  return ok();
}

int qdec_adaptor_run(qdec_adaptor* a, const float* frames_dev, int32_t n_frames, float* out_dev) {
  if (!a) return fail(QDEC_E_INVALID, "adaptor is NULL");
  if (n_frames < 1) return fail(QDEC_E_INVALID, "n_frames %d < 1", n_frames);
  const qdec_adaptor_config& c = a->c;
  const int T = n_frames, D = c.dim, F = c.ffn_dim;
  if (int e = check_dev(frames_dev, (size_t)T * c.enc_dim * sizeof(float), "frames_dev")) return e;
  if (int e = check_dev(out_dev, (size_t)T * D * sizeof(float), "out_dev")) return e;
  {
    const char *f0 = (const char*)frames_dev, *f1 = f0 + (size_t)T * c.enc_dim * sizeof(float);
    const char *o0 = (const char*)out_dev, *o1 = o0 + (size_t)T * D * sizeof(float);
    if (f0 < o1 && o0 < f1) return fail(QDEC_E_INVALID, "out_dev overlaps frames_dev");
  }
  if (int e = ensure_adaptor(a, T)) return e;
  hipStream_t st = a->stream;
  uint16_t *A0 = a->A0, *A1 = a->A1;
  const Dims ad = adaptor_dims(c);
  LAUNCH(launch_rms_split(frames_dev, T, c.enc_dim, nullptr, 0.f, A0, A1, st));
  SplitK* sk = &a->split.sk;
  LAUNCH(launch_gemm(true, EPI_RELU, A0, A1, T, c.enc_dim, a->w1, c.mid_dim, a->H, c.mid_dim, st, a->b1, sk));
  LAUNCH(launch_rms_split(a->H, T, c.mid_dim, nullptr, 0.f, A0, A1, st));
  LAUNCH(launch_gemm(true, EPI_STORE, A0, A1, T, c.mid_dim, a->w2, D, out_dev, D, st, a->b2, sk));
  for (const qdec_adaptor::Block& k : a->blocks) {
    LAUNCH(launch_ln_split(out_dev, T, D, k.n1g, k.n1b, c.ln_eps, A0, A1, st));
    LAUNCH(launch_gemm(true, EPI_STORE, A0, A1, T, D, k.wqkv, 3 * D, a->QKV, 3 * D, st, k.bqkv, sk));
    LAUNCH(launch_attn_prefill(ad, a->QKV, T, nullptr, a->kv, st, A0, A1, false, sk));
    LAUNCH(launch_gemm(true, EPI_RESID, A0, A1, T, D, k.wo, D, out_dev, D, st, k.bo, sk));
    LAUNCH(launch_ln_split(out_dev, T, D, k.n2g, k.n2b, c.ln_eps, A0, A1, st));
    LAUNCH(launch_gemm(true, EPI_RELU, A0, A1, T, D, k.fc1, F, a->H, F, st, k.bf1, sk));
    LAUNCH(launch_rms_split(a->H, T, F, nullptr, 0.f, A0, A1, st));
    LAUNCH(launch_gemm(true, EPI_RESID, A0, A1, T, F, k.fc2, D, out_dev, D, st, k.bf2, sk));
  }
  return ok();
}

void qdec_adaptor_destroy(qdec_adaptor* a) { free_adaptor(a); }

}  // extern "C"

// ================================================================= encoder
// The audio frontend and the SAN-M speech encoder (audio.cpp "Fun-ASR-Nano
// Native Runtime Implementation Plan", Tasks 2-4; transcribe.cpp "Forward map
// - funasr_nano", tables "Frontend" and "Encoder"). The frontend kernels run
// in float64; the 70 blocks reuse the prefill kernels: LayerNorm written as a
// bf16 hi/lo operand, the MFMA GEMMs with bias / ReLU / residual epilogues,
// the matrix-core attention without the causal mask, plus the FSMN kernel
// that adds v + conv(v) into the residual stream ahead of the O projection's
// residual epilogue.

struct qdec_encoder {
  qdec_encoder_config c{};
  hipStream_t stream = nullptr;
  int in_dim = 0, in_pad = 0;  // LFR row width and the stem's GEMM operand pitch (multiple of 32)
  struct Block {
    uint16_t* wqkv = nullptr;  // [3 dim, in_pad] (owned): q rows, k rows, v rows
    const uint16_t *wo = nullptr, *ffn1 = nullptr, *ffn2 = nullptr;
    float *bqkv = nullptr, *bo = nullptr, *n1g = nullptr, *n1b = nullptr, *n2g = nullptr, *n2b = nullptr;
    float *bf1 = nullptr, *bf2 = nullptr, *taps = nullptr;
  };
  std::vector<Block> blocks;
  float* vecs = nullptr;  // biases, norm vectors and FSMN taps, fp32
  float *an_g = nullptr, *an_b = nullptr, *tn_g = nullptr, *tn_b = nullptr;
  double* tab = nullptr;  // frontend tables and the PE frequencies, fp64
  int* mel_range = nullptr;
  const double* inv_freq = nullptr;
  FrontTables ft{};
  SplitKBuf split;  // split-K workspace of the GEMMs
  // scratch for up to cap_rows LFR rows (cap_rows * lfr_n + lfr_m frames)
  int cap_rows = 0;
  float* fb = nullptr;
  float* x0 = nullptr;
  float* X = nullptr;
  float* QKV = nullptr;
  float* H = nullptr;
  uint16_t* A0 = nullptr;
  uint16_t* A1 = nullptr;
  uint16_t* kv[4] = {nullptr, nullptr, nullptr, nullptr};
};

namespace {

void free_encoder_scratch(qdec_encoder* e) {
  for (void* p : {(void*)e->fb, (void*)e->x0, (void*)e->X, (void*)e->QKV, (void*)e->H, (void*)e->A0, (void*)e->A1,
                  (void*)e->kv[0], (void*)e->kv[1], (void*)e->kv[2], (void*)e->kv[3]})
    if (p) (void)dfree(p);
  e->fb = e->x0 = e->X = e->QKV = e->H = nullptr;
  e->A0 = e->A1 = nullptr;
  for (auto& k : e->kv) k = nullptr;
  e->cap_rows = 0;
}

void free_encoder(qdec_encoder* e) {
  if (!e) return;
  (void)hipStreamSynchronize(e->stream);
  free_encoder_scratch(e);
  for (auto& b : e->blocks)
    if (b.wqkv) (void)dfree(b.wqkv);
  for (void* p : {(void*)e->vecs, (void*)e->tab, (void*)e->mel_range})
    if (p) (void)dfree(p);
  free_splitk(&e->split);
  delete e;
}

int ensure_encoder(qdec_encoder* e, int rows) {
  if (rows <= e->cap_rows) return QDEC_OK;
  free_encoder_scratch(e);
  const qdec_encoder_config& c = e->c;
  const size_t R = (size_t)rows, frames = R * c.lfr_n + c.lfr_m;
  const size_t wide = (size_t)std::max(std::max(e->in_pad, c.dim), c.ffn_dim);
  const size_t Tp = (size_t)kv_split_pad(rows);
  int r;
  if ((r = dev_alloc(&e->fb, frames * kMels, "fbank frames")) ||
      (r = dev_alloc(&e->x0, R * e->in_dim, "encoder input rows")) ||
      (r = dev_alloc(&e->X, R * c.dim, "encoder residual stream")) ||
      (r = dev_alloc(&e->QKV, R * 3 * c.dim, "encoder qkv")) || (r = dev_alloc(&e->H, R * c.ffn_dim, "encoder ffn")) ||
      (r = dev_alloc(&e->A0, R * wide, "encoder operand")) || (r = dev_alloc(&e->A1, R * wide, "encoder operand")) ||
      (r = dev_alloc(&e->kv[0], R * c.dim, "encoder K")) || (r = dev_alloc(&e->kv[1], R * c.dim, "encoder K")) ||
      (r = dev_alloc(&e->kv[2], Tp * c.dim, "encoder V")) || (r = dev_alloc(&e->kv[3], Tp * c.dim, "encoder V"))) {
    free_encoder_scratch(e);
    return r;
  }
  e->cap_rows = rows;
  return QDEC_OK;
}

int frames_of(int64_t n) { return n < kFrameLen ? 0 : (int)(1 + (n - kFrameLen) / kFrameShift); }

// The encoder blocks over the rows in e->x0, result into out.
int encoder_blocks(qdec_encoder* e, int T, float* out) {
  const qdec_encoder_config& c = e->c;
  const int D = c.dim, F = c.ffn_dim;
  hipStream_t st = e->stream;
  uint16_t *A0 = e->A0, *A1 = e->A1;
  const Dims ad{1, D, c.n_head, c.n_head, 128, 0, 0, 0.f};
  SplitK* sk = &e->split.sk;
  for (size_t b = 0; b < e->blocks.size(); ++b) {
    const qdec_encoder::Block& k = e->blocks[b];
    const bool stem = b == 0;
    if (stem)
      LAUNCH(launch_ln_split(e->x0, T, e->in_dim, k.n1g, k.n1b, c.ln_eps, A0, A1, st, e->in_pad));
    else
      LAUNCH(launch_ln_split(e->X, T, D, k.n1g, k.n1b, c.ln_eps, A0, A1, st));
    LAUNCH(launch_gemm(true, EPI_STORE, A0, A1, T, stem ? e->in_pad : D, k.wqkv, 3 * D, e->QKV, 3 * D, st, k.bqkv,
                       sk));
    LAUNCH(launch_attn_prefill(ad, e->QKV, T, nullptr, e->kv, st, A0, A1, false, sk));
    LAUNCH(launch_fsmn(e->QKV, 3 * D, T, D, c.fsmn_kernel, k.taps, !stem, e->X, st));
    LAUNCH(launch_gemm(true, EPI_RESID, A0, A1, T, D, k.wo, D, e->X, D, st, k.bo, sk));
    LAUNCH(launch_ln_split(e->X, T, D, k.n2g, k.n2b, c.ln_eps, A0, A1, st));
    LAUNCH(launch_gemm(true, EPI_RELU, A0, A1, T, D, k.ffn1, F, e->H, F, st, k.bf1, sk));
    LAUNCH(launch_rms_split(e->H, T, F, nullptr, 0.f, A0, A1, st));
    LAUNCH(launch_gemm(true, EPI_RESID, A0, A1, T, F, k.ffn2, D, e->X, D, st, k.bf2, sk));
    if ((int)b == c.n_main) LAUNCH(launch_ln_apply(e->X, T, D, e->an_g, e->an_b, c.ln_eps, e->X, st));
  }
  LAUNCH(launch_ln_apply(e->X, T, D, e->tn_g, e->tn_b, c.ln_eps, out, st));
  return QDEC_OK;
}

// Frontend of n samples: fbank frames into e->fb, then the LFR rows into
// lfr (optional) and the encoder input rows into e->x0 (when x0 is set).
int run_frontend(qdec_encoder* e, const float* pcm, int64_t n, float* lfr, bool x0) {
  const qdec_encoder_config& c = e->c;
  const int frames = frames_of(n), rows = (frames + c.lfr_n - 1) / c.lfr_n;
  LAUNCH(launch_fbank(pcm, frames, e->ft, e->fb, e->stream));
  LAUNCH(launch_lfr_embed(e->fb, frames, kMels, c.lfr_m, c.lfr_n, sqrtf((float)c.dim), e->inv_freq, lfr,
                          x0 ? e->x0 : nullptr, rows, e->stream));
  return QDEC_OK;
}

int check_pcm(qdec_encoder* e, const float* pcm, int64_t n, int* rows) {
  if (!e) return fail(QDEC_E_INVALID, "encoder is NULL");
  if (n < kFrameLen) return fail(QDEC_E_INVALID, "%lld samples: at least %d are needed", (long long)n, kFrameLen);
  const int64_t frames = 1 + (n - kFrameLen) / kFrameShift;
  if (frames > (int64_t)e->c.lfr_n * 65536) return fail(QDEC_E_INVALID, "input longer than 65536 LFR rows");
  if (int r = check_dev(pcm, (size_t)n * sizeof(float), "pcm_dev")) return r;
  *rows = (int)((frames + e->c.lfr_n - 1) / e->c.lfr_n);
  return ensure_encoder(e, *rows);
}

}  // namespace

extern "C" {

int qdec_encoder_create(const qdec_encoder_config* cfg, const qdec_encoder_weights* w, void* hip_stream,
                        qdec_encoder** out) {
  if (!out) return fail(QDEC_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(QDEC_E_INVALID, "config is NULL");
  const qdec_encoder_config& c = *cfg;
  if (c.weight_dtype != QDEC_BF16) return fail(QDEC_E_INVALID, "the encoder takes bf16 weights");
  if (c.n_mels != kMels) return fail(QDEC_E_INVALID, "n_mels %d: the frontend computes %d", c.n_mels, kMels);
  if (c.lfr_m < 1 || c.lfr_m > 15 || c.lfr_m % 2 == 0 || c.lfr_n < 1 || c.lfr_n > 15)
    return fail(QDEC_E_INVALID, "lfr_m %d (odd, 1 .. 15) or lfr_n %d (1 .. 15)", c.lfr_m, c.lfr_n);
  if (c.n_head < 1 || c.n_head > 16 || c.dim != c.n_head * 128)
    return fail(QDEC_E_INVALID, "dim %d must be n_head (%d) * 128", c.dim, c.n_head);
  if (c.ffn_dim < 128 || c.ffn_dim > 8192 || c.ffn_dim % 128)
    return fail(QDEC_E_INVALID, "ffn_dim %d must be a multiple of 128 in [128, 8192]", c.ffn_dim);
  if (c.fsmn_kernel < 1 || c.fsmn_kernel > 31 || c.fsmn_kernel % 2 == 0)
    return fail(QDEC_E_INVALID, "fsmn_kernel %d must be odd in [1, 31]", c.fsmn_kernel);
  if (c.n_main < 0 || c.n_main > 127 || c.n_tp < 0 || c.n_tp > 127)
    return fail(QDEC_E_INVALID, "n_main %d / n_tp %d outside 0 .. 127", c.n_main, c.n_tp);
  if (!(c.ln_eps > 0.f) || !std::isfinite(c.ln_eps)) return fail(QDEC_E_INVALID, "ln_eps must be > 0");
  if (!w || !w->block || !w->after_norm_g || !w->after_norm_b || !w->tp_norm_g || !w->tp_norm_b)
    return fail(QDEC_E_INVALID, "encoder weights incomplete");
  const int nb = 1 + c.n_main + c.n_tp;
  const size_t D = c.dim, F = c.ffn_dim, K = c.fsmn_kernel, W = (size_t)kMels * c.lfr_m;
  for (int b = 0; b < nb; ++b) {
    const void* const* t = w->block + (size_t)b * QDEC_EB_PER_BLOCK;
    const size_t in = b == 0 ? W : D;
    const size_t n[QDEC_EB_PER_BLOCK] = {in, in, D * in, D, D * in, D, D * in, D, D * K, D * D, D, D, D, F * D, F,
                                         D * F, D};
    for (int i = 0; i < QDEC_EB_PER_BLOCK; ++i) {
      char what[48];
      snprintf(what, sizeof what, "block %d tensor %d", b, i);
      if (int r = check_dev(t[i], n[i] * 2, what)) return r;
    }
  }
  for (const void* p : {w->after_norm_g, w->after_norm_b, w->tp_norm_g, w->tp_norm_b})
    if (int r = check_dev(p, D * 2, "final norm vector")) return r;

  qdec_encoder* e = new (std::nothrow) qdec_encoder();
  if (!e) return fail(QDEC_E_OOM, "host allocation failed");
  e->c = c;
  e->stream = (hipStream_t)hip_stream;
  e->in_dim = (int)W;
  e->in_pad = (int)((W + 31) / 32 * 32);
  hipStream_t st = e->stream;
  auto fail_dev = [&](const char* what, hipError_t he) {
    const int r = fail(QDEC_E_DEVICE, "%s: %s", what, hipGetErrorString(he));
    free_encoder(e);
    return r;
  };
  // fp32 vectors: per block 2 norm1 (in wide), qkv, o, 2 norm2, ffn biases, taps
  const size_t per_block = 2 * std::max(W, D) + 3 * D + D + 2 * D + F + D + D * K;
  const size_t nvec = (size_t)nb * per_block + 4 * D;
  if (int r = dev_alloc(&e->vecs, nvec, "encoder vectors")) {
    free_encoder(e);
    return r;
  }
  if (int r = alloc_splitk(&e->split)) {
    free_encoder(e);
    return r;
  }
  hipError_t he;
  float* v = e->vecs;
  e->blocks.resize(nb);
  for (int b = 0; b < nb; ++b) {
    const void* const* t = w->block + (size_t)b * QDEC_EB_PER_BLOCK;
    qdec_encoder::Block& k = e->blocks[b];
    const size_t in = b == 0 ? W : D, pitch = b == 0 ? (size_t)e->in_pad : D;
    if (int r = dev_alloc(&k.wqkv, 3 * D * pitch, "encoder wqkv")) {
      free_encoder(e);
      return r;
    }
    if ((he = hipMemsetAsync(k.wqkv, 0, 3 * D * pitch * 2, st))) return fail_dev("clear wqkv", he);
    const int srcs[3] = {QDEC_EB_Q_W, QDEC_EB_K_W, QDEC_EB_V_W};
    for (int j = 0; j < 3; ++j)
      if ((he = hipMemcpy2DAsync(k.wqkv + j * D * pitch, pitch * 2, t[srcs[j]], in * 2, in * 2, D,
                                 hipMemcpyDeviceToDevice, st)))
        return fail_dev("pack wqkv", he);
    k.wo = (const uint16_t*)t[QDEC_EB_O_W];
    k.ffn1 = (const uint16_t*)t[QDEC_EB_FFN1_W];
    k.ffn2 = (const uint16_t*)t[QDEC_EB_FFN2_W];
    k.n1g = v;
    k.n1b = v + in;
    v += 2 * std::max(W, D);
    k.bqkv = v;
    k.bo = v + 3 * D;
    k.n2g = v + 4 * D;
    k.n2b = v + 5 * D;
    k.bf2 = v + 6 * D;
    k.bf1 = v + 7 * D;
    k.taps = v + 7 * D + F;
    v += 3 * D + D + 2 * D + D + F + D * K;
    const struct {
      int idx;
      float* dst;
      size_t n;
    } vecs[] = {{QDEC_EB_NORM1_G, k.n1g, in}, {QDEC_EB_NORM1_B, k.n1b, in},  {QDEC_EB_Q_B, k.bqkv, D},
                {QDEC_EB_K_B, k.bqkv + D, D}, {QDEC_EB_V_B, k.bqkv + 2 * D, D}, {QDEC_EB_O_B, k.bo, D},
                {QDEC_EB_NORM2_G, k.n2g, D},  {QDEC_EB_NORM2_B, k.n2b, D},   {QDEC_EB_FFN2_B, k.bf2, D},
                {QDEC_EB_FFN1_B, k.bf1, F},   {QDEC_EB_FSMN_W, k.taps, D * K}};
    for (const auto& x : vecs)
      if ((he = launch_to_f32(t[x.idx], true, x.n, x.dst, st))) return fail_dev("encoder vector", he);
  }
  e->an_g = v;
  e->an_b = v + D;
  e->tn_g = v + 2 * D;
  e->tn_b = v + 3 * D;
  if ((he = launch_to_f32(w->after_norm_g, true, D, e->an_g, st)) ||
      (he = launch_to_f32(w->after_norm_b, true, D, e->an_b, st)) ||
      (he = launch_to_f32(w->tp_norm_g, true, D, e->tn_g, st)) ||
      (he = launch_to_f32(w->tp_norm_b, true, D, e->tn_b, st)))
    return fail_dev("final norms", he);

  // frontend tables, computed here in double: Hamming window, FFT twiddles,
  // the mel triangles (HTK mel 1127 ln(1 + f / 700), 82 edges equally spaced
  // in mel from 20 Hz to 8000 Hz, bins at 31.25 Hz) and the PE frequencies
  constexpr int kBins = 256;
  const size_t n_tab = kFrameLen + 2 * kBins + (size_t)kMels * kBins + W / 2;
  std::vector<double> h(n_tab, 0.0);
  std::vector<int> range(2 * kMels, 0);
  double* hw = h.data();
  double* htr = hw + kFrameLen;
  double* hti = htr + kBins;
  double* hm = hti + kBins;
  double* hf = hm + (size_t)kMels * kBins;
  const double pi = 3.14159265358979323846;
  for (int i = 0; i < kFrameLen; ++i) hw[i] = 0.54 - 0.46 * std::cos(2.0 * pi * i / (kFrameLen - 1));
  for (int k = 0; k < kBins; ++k) {
    htr[k] = std::cos(2.0 * pi * k / (2 * kBins));
    hti[k] = -std::sin(2.0 * pi * k / (2 * kBins));
  }
  auto to_mel = [](double f) { return 1127.0 * std::log(1.0 + f / 700.0); };
  const double m_lo = to_mel(20.0), m_hi = to_mel(8000.0), step = (m_hi - m_lo) / (kMels + 1);
  for (int j = 0; j < kMels; ++j) {
    const double left = m_lo + j * step, centre = m_lo + (j + 1) * step, right = m_lo + (j + 2) * step;
    int lo = kBins, hi = 0;
    for (int k = 0; k < kBins; ++k) {
      const double m = to_mel(k * 16000.0 / (2 * kBins));
      double wgt = 0.0;
      if (m > left && m < right) wgt = m <= centre ? (m - left) / (centre - left) : (right - m) / (right - centre);
      hm[(size_t)j * kBins + k] = wgt;
      if (wgt != 0.0) {
        lo = std::min(lo, k);
        hi = k + 1;
      }
    }
    range[j] = lo < hi ? lo : 0;
    range[kMels + j] = lo < hi ? hi : 0;
  }
  for (size_t i = 0; i < W / 2; ++i) hf[i] = 1.0 / std::pow(10000.0, 2.0 * (double)i / (double)W);
  if (int r = dev_alloc(&e->tab, n_tab, "frontend tables")) {
    free_encoder(e);
    return r;
  }
  if (int r = dev_alloc(&e->mel_range, 2 * kMels, "mel ranges")) {
    free_encoder(e);
    return r;
  }
  if ((he = hipMemcpyAsync(e->tab, h.data(), n_tab * sizeof(double), hipMemcpyHostToDevice, st)) ||
      (he = hipMemcpyAsync(e->mel_range, range.data(), range.size() * sizeof(int), hipMemcpyHostToDevice, st)))
    return fail_dev("frontend tables", he);
  e->ft = FrontTables{e->tab, e->tab + kFrameLen, e->tab + kFrameLen + kBins, e->tab + kFrameLen + 2 * kBins,
                      e->mel_range, e->mel_range + kMels};
  e->inv_freq = e->tab + kFrameLen + 2 * kBins + (size_t)kMels * kBins;
  // the host vectors are read by the copies above: wait before they go
  if ((he = hipStreamSynchronize(st))) return fail_dev("encoder packing", he);
  *out = e;
  return ok();
}

int32_t qdec_encoder_rows(const qdec_encoder* e, int64_t n_samples) {
  if (!e) return 0;
  const int f = frames_of(n_samples);
  return (f + e->c.lfr_n - 1) / e->c.lfr_n;
}

int qdec_frontend_run(qdec_encoder* e, const float* pcm_dev, int64_t n_samples, float* lfr_dev) {
  int rows = 0;
  if (int r = check_pcm(e, pcm_dev, n_samples, &rows)) return r;
  if (int r = check_dev(lfr_dev, (size_t)rows * e->in_dim * sizeof(float), "lfr_dev")) return r;
  if (int r = run_frontend(e, pcm_dev, n_samples, lfr_dev, false)) return r;
  return ok();
}

int qdec_encoder_forward(qdec_encoder* e, const float* lfr_dev, int32_t n_rows, float* out_dev) {
  if (!e) return fail(QDEC_E_INVALID, "encoder is NULL");
  if (n_rows < 1 || n_rows > 65536) return fail(QDEC_E_INVALID, "n_rows %d outside 1 .. 65536", n_rows);
  if (int r = check_dev(lfr_dev, (size_t)n_rows * e->in_dim * sizeof(float), "lfr_dev")) return r;
  if (int r = check_dev(out_dev, (size_t)n_rows * e->c.dim * sizeof(float), "out_dev")) return r;
  if (int r = ensure_encoder(e, n_rows)) return r;
  // the rows themselves as one-frame LFR rows: x0 = rows * sqrt(dim) + PE
  LAUNCH(launch_lfr_embed(lfr_dev, n_rows, e->in_dim, 1, 1, sqrtf((float)e->c.dim), e->inv_freq, nullptr, e->x0,
                          n_rows, e->stream));
  if (int r = encoder_blocks(e, n_rows, out_dev)) return r;
  return ok();
}

int qdec_encoder_run(qdec_encoder* e, const float* pcm_dev, int64_t n_samples, float* out_dev) {
  int rows = 0;
  if (int r = check_pcm(e, pcm_dev, n_samples, &rows)) return r;
  if (int r = check_dev(out_dev, (size_t)rows * e->c.dim * sizeof(float), "out_dev")) return r;
  if (int r = run_frontend(e, pcm_dev, n_samples, nullptr, true)) return r;
  if (int r = encoder_blocks(e, rows, out_dev)) return r;
  return ok();
}

void qdec_encoder_destroy(qdec_encoder* e) { free_encoder(e); }

}  // extern "C"
