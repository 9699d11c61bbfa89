/* Host-side checks of the qdec C ABI for a build of the host code under
 * AddressSanitizer and UndefinedBehaviorSanitizer (test_host_sanitizers.py).
 * Every call here fails before it touches a GPU: bad configs, NULL handles
 * and buffers, host memory passed where device memory is required, and
 * error strings kept per thread. Exits 0 when every return code is the
 * documented one; the sanitizers abort the process on any invalid access,
 * leak or undefined operation along the way. */
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qdec.h"

static int failures = 0;

#define EXPECT(call, code)                                                                   \
  do {                                                                                       \
    const int r_ = (call);                                                                   \
    if (r_ != (code)) {                                                                      \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, \
              r_, (int)(code), qdec_last_error());                                           \
      ++failures;                                                                            \
    } else if ((code) != QDEC_OK && qdec_last_error()[0] == '\0') {                          \
      fprintf(stderr, "%s:%d: %s gave no error text\n", __FILE__, __LINE__, #call);          \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

static qdec_config good_config(void) {
  qdec_config c;
  memset(&c, 0, sizeof c);
  c.n_layer = 2;
  c.hidden = 128;
  c.n_q_head = 4;
  c.n_kv_head = 2;
  c.head_dim = 32;
  c.ffn = 384;
  c.vocab = 1024;
  c.rms_eps = 1e-6f;
  c.rope_theta = 1e6f;
  c.weight_dtype = QDEC_BF16;
  c.tied = 1;
  return c;
}

static void model_checks(void) {
  qdec_model* m = (qdec_model*)0x1;
  const void* null_layers[2 * QDEC_W_PER_LAYER] = {0};
  qdec_weights w = {0, 0, null_layers};
  qdec_config c = good_config();
  EXPECT(qdec_create(&c, &w, 0, 0), QDEC_E_INVALID);  /* out is NULL */
  EXPECT(qdec_create(0, &w, 0, &m), QDEC_E_INVALID);  /* config is NULL */
  if (m) {
    fprintf(stderr, "qdec_create left *out set after a failure\n");
    ++failures;
  }
  EXPECT(qdec_create(&c, 0, 0, &m), QDEC_E_INVALID);
  EXPECT(qdec_create(&c, &w, 0, &m), QDEC_E_INVALID); /* weights incomplete */

  /* each field out of range in turn */
  struct { int field; int value; } bad[] = {
      {0, 0}, {1, 100}, {1, 0}, {1, 2048}, {4, 48}, {4, 256}, {3, 3}, {5, 100}, {5, 96}, {5, 8256},
      {6, 1}, {7, 0}, {8, 7}};
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    qdec_config b = good_config();
    int32_t* f[] = {&b.n_layer, &b.hidden, &b.n_q_head, &b.n_kv_head, &b.head_dim, &b.ffn, &b.vocab,
                    &b.tied, &b.weight_dtype};
    *f[bad[i].field] = bad[i].value;
    EXPECT(qdec_create(&b, &w, 0, &m), QDEC_E_INVALID);
  }
  qdec_config e = good_config();
  e.rms_eps = 0.f;
  EXPECT(qdec_create(&e, &w, 0, &m), QDEC_E_INVALID);
  e = good_config();
  e.rope_theta = 0.5f;
  EXPECT(qdec_create(&e, &w, 0, &m), QDEC_E_INVALID);
  e = good_config();
  e.weight_dtype = QDEC_Q8_0; /* ffn 384 is not whole 256-input slices */
  EXPECT(qdec_create(&e, &w, 0, &m), QDEC_E_INVALID);

  /* host memory where device memory belongs: rejected by the pointer check */
  float* host = (float*)calloc((size_t)1024 * 128, sizeof(float));
  const void* host_layers[2 * QDEC_W_PER_LAYER];
  for (int i = 0; i < 2 * QDEC_W_PER_LAYER; ++i) host_layers[i] = host;
  qdec_weights hw = {host, host, host_layers};
  EXPECT(qdec_create(&c, &hw, 0, &m), QDEC_E_INVALID);
  free(host);

  /* NULL handles */
  EXPECT(qdec_destroy(0), QDEC_OK);
  qdec_state_destroy(0);
  if (qdec_state_pos(0) != -1) {
    fprintf(stderr, "qdec_state_pos(NULL) != -1\n");
    ++failures;
  }
  qdec_state* s = (qdec_state*)0x1;
  EXPECT(qdec_state_create(0, 16, &s), QDEC_E_INVALID);
  EXPECT(qdec_state_create(0, 16, 0), QDEC_E_INVALID);
  int32_t ids[2] = {1, 2};
  EXPECT(qdec_prefill(0, ids, 2, 0, 0, 0, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_decode_step(0, 1, 0, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_decode_step_dev(0, 0, 0, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_decode_greedy(0, 0, 0, 1, 0, 0), QDEC_E_INVALID);
  qdec_state* states[17] = {0};
  int32_t toks[17] = {0};
  EXPECT(qdec_decode_batch(states, 0, toks, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_decode_batch(states, 17, toks, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_decode_batch(0, 1, toks, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_decode_batch(states, 1, toks, 0, 0), QDEC_E_INVALID);
  EXPECT(qdec_clone_state(0, &s), QDEC_E_INVALID);
  EXPECT(qdec_model_status(0), QDEC_E_INVALID);
  qdec_sampling p = {1.0f, 10, 1.0f, 1.0f};
  float u = 0.5f;
  EXPECT(qdec_sample(0, 0, 1, &p, 0, 0, &u, 0), QDEC_E_INVALID);
  EXPECT(qdec_sample_noalloc(0, 0, 1, &p, 0, 0, &u, 0), QDEC_E_INVALID);
}

static qdec_adaptor_config adaptor_config(void) {
  qdec_adaptor_config c = {512, 2048, 1024, 256, 2, 8, 1e-12f, QDEC_BF16};
  return c;
}

static void adaptor_checks(void) {
  qdec_adaptor* a = 0;
  qdec_adaptor_weights w = {0, 0, 0, 0, 0};
  qdec_adaptor_config c = adaptor_config();
  EXPECT(qdec_adaptor_create(&c, &w, 0, &a), QDEC_E_INVALID); /* weights incomplete */
  EXPECT(qdec_adaptor_create(0, &w, 0, &a), QDEC_E_INVALID);
  EXPECT(qdec_adaptor_create(&c, &w, 0, 0), QDEC_E_INVALID);
  for (int i = 0; i < 8; ++i) {
    qdec_adaptor_config b = adaptor_config();
    switch (i) {
      case 0: b.weight_dtype = QDEC_F32; break;
      case 1: b.enc_dim = 100; break;
      case 2: b.mid_dim = 2000; break;
      case 3: b.ffn_dim = 200; break;
      case 4: b.dim = 1000; break;
      case 5: b.n_block = 0; break;
      case 6: b.n_block = 9; break;
      default: b.ln_eps = 0.f; break;
    }
    EXPECT(qdec_adaptor_create(&b, &w, 0, &a), QDEC_E_INVALID);
  }
  float host[64];
  EXPECT(qdec_adaptor_run(0, host, 4, host), QDEC_E_INVALID);
  qdec_adaptor_destroy(0);
}

static qdec_encoder_config encoder_config(void) {
  qdec_encoder_config c = {80, 7, 6, 512, 4, 2048, 11, 49, 20, 1e-12f, QDEC_BF16};
  return c;
}

static void encoder_checks(void) {
  qdec_encoder* e = 0;
  qdec_encoder_weights w = {0, 0, 0, 0, 0};
  qdec_encoder_config c = encoder_config();
  EXPECT(qdec_encoder_create(&c, &w, 0, &e), QDEC_E_INVALID);
  EXPECT(qdec_encoder_create(0, &w, 0, &e), QDEC_E_INVALID);
  for (int i = 0; i < 11; ++i) {
    qdec_encoder_config b = encoder_config();
    switch (i) {
      case 0: b.weight_dtype = QDEC_F32; break;
      case 1: b.n_mels = 64; break;
      case 2: b.lfr_m = 6; break;
      case 3: b.lfr_m = 17; break;
      case 4: b.lfr_n = 0; break;
      case 5: b.dim = 500; break;
      case 6: b.ffn_dim = 1000; break;
      case 7: b.fsmn_kernel = 10; break;
      case 8: b.n_main = -1; break;
      case 9: b.n_tp = 128; break;
      default: b.ln_eps = 0.f; break;
    }
    EXPECT(qdec_encoder_create(&b, &w, 0, &e), QDEC_E_INVALID);
  }
  float host[64];
  EXPECT(qdec_encoder_run(0, host, 16000, host), QDEC_E_INVALID);
  EXPECT(qdec_frontend_run(0, host, 16000, host), QDEC_E_INVALID);
  EXPECT(qdec_encoder_forward(0, host, 4, host), QDEC_E_INVALID);
  EXPECT(qdec_encoder_rows(0, 16000), 0);
  qdec_encoder_destroy(0);
}

/* qdec_last_error is per thread: a second thread's failures (a different
 * message) do not change this thread's text */
static void* other_thread(void* arg) {
  (void)arg;
  for (int i = 0; i < 200; ++i) {
    if (qdec_state_create(0, 16, 0) != QDEC_E_INVALID || strstr(qdec_last_error(), "out") == 0) return (void*)1;
  }
  return 0;
}

static void thread_checks(void) {
  qdec_state* s = 0;
  EXPECT(qdec_state_create((qdec_model*)0, 0, &s), QDEC_E_INVALID);
  char mine[512];
  snprintf(mine, sizeof mine, "%s", qdec_last_error());
  pthread_t t;
  void* r = 0;
  if (pthread_create(&t, 0, other_thread, 0) != 0 || pthread_join(t, &r) != 0 || r != 0) {
    fprintf(stderr, "second thread failed\n");
    ++failures;
  }
  if (strcmp(mine, qdec_last_error()) != 0) {
    fprintf(stderr, "error text changed by another thread: '%s' -> '%s'\n", mine, qdec_last_error());
    ++failures;
  }
}

int main(void) {
  model_checks();
  adaptor_checks();
  encoder_checks();
  thread_checks();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
