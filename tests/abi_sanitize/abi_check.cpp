/* The library's host-side logic under AddressSanitizer and UndefinedBehaviorSanitizer
 * (host code only is instrumented; built by tests/abi_sanitize/sanitized_build.py).
 *
 *   abi_check host    the ledger (admission, shrink, the 97/3/100 capacity edge,
 *                     rewind, every error, no state change on error), rope-width
 *                     resolution, and every argument and geometry check of
 *                     eagle3_load / eagle3_trunk_load / eagle3_verify_attention /
 *                     eagle3_generate that fails before any device work; runs
 *                     without a GPU.
 *   abi_check device  allocation failure injected at every device allocation of a
 *                     small eagle3_load and eagle3_trunk_load in turn: each must
 *                     return EAGLE3_E_OOM, leave the handle NULL and release all it
 *                     had allocated (the library's count of live device and pinned
 *                     allocations, eagle3_test_live_allocations, is back where it
 *                     was; LeakSanitizer checks the host side at exit); the sweep
 *                     ends with a clean load and free.  Needs a GPU.
 * Exit status 0 when every check holds; each failed check prints a line.
 * (pegainfer PR #707, review: cleanup on failure, cache-edge and abort cases.) */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <sanitizer/lsan_interface.h>

#include "eagle3.h"
#include "eagle3_ledger.h"
#include "eagle3_testing.h"
#include "eagle3_trunk.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* a small drafter geometry: n 256, 4/2 heads x 64, ff 768, vocab 1024/4096 */
static eagle3_config small_config(void) {
  eagle3_config c;
  memset(&c, 0, sizeof c);
  c.n_embd = 256; c.n_head = 4; c.n_head_kv = 2; c.head_dim = 64; c.n_ff = 768;
  c.draft_vocab = 1024; c.target_vocab = 4096; c.n_aux = 3; c.rope_dim = 64;
  c.rope_theta = 1e4f; c.rms_eps = 1e-6f; c.max_ctx = 128; c.max_gamma = 8; c.max_seqs = 2;
  c.kv_dtype = EAGLE3_KV_F32; c.weight_format = EAGLE3_WEIGHTS_BF16; c.append_act = EAGLE3_APPEND_DEFAULT;
  c.token_table = EAGLE3_TABLE_DEFAULT;
  return c;
}

static void fill_shapes(const eagle3_config* c, eagle3_weights* w) {
  const int64_t n = c->n_embd, qd = (int64_t)c->n_head * c->head_dim, kvd = (int64_t)c->n_head_kv * c->head_dim;
  const int64_t s[14][2] = {{n, 3 * n}, {n, 1}, {n, 1}, {qd, 2 * n}, {kvd, 2 * n}, {kvd, 2 * n}, {n, qd},
                            {n, 1}, {c->n_ff, n}, {c->n_ff, n}, {n, c->n_ff}, {n, 1}, {c->draft_vocab, n},
                            {c->target_vocab, n}};
  memcpy(w->shape, s, sizeof s);
}

static void check_ledger(void) {
  eagle3_ledger* l = NULL;
  int32_t g = -1, c = -1, sp = -1;
  CHECK(eagle3_ledger_create(0, 1, 3, &l) == EAGLE3_E_INVAL && l == NULL);
  CHECK(eagle3_ledger_create(100, 2, 3, NULL) == EAGLE3_E_INVAL);
  CHECK(eagle3_ledger_create(100, 2, 3, &l) == EAGLE3_OK && l != NULL);
  if (!l) return;
  /* the 97/3/100 edge: a chain of 3 at 97, full acceptance commits 4 rows */
  CHECK(eagle3_ledger_prefill(l, 0, 97, 0) == EAGLE3_OK);
  CHECK(eagle3_ledger_prefill(l, 0, 4, 0) == EAGLE3_E_CAPACITY);
  CHECK(eagle3_ledger_len(l, 0, &c, &sp) == EAGLE3_OK && c == 97 && sp == 0);
  CHECK(eagle3_ledger_rebuild(l, 0, 0, 0) == EAGLE3_E_STATE);      /* no chain round yet */
  CHECK(eagle3_ledger_chain(l, 0, 3, 0, &g) == EAGLE3_OK && g == 3);
  CHECK(eagle3_ledger_rebuild(l, 0, 4, 0) == EAGLE3_E_INVAL);      /* a > gamma_eff */
  CHECK(eagle3_ledger_len(l, 0, &c, &sp) == EAGLE3_OK && c == 97 && sp == 0);
  CHECK(eagle3_ledger_rebuild(l, 0, 3, 0) == EAGLE3_OK);
  CHECK(eagle3_ledger_len(l, 0, &c, &sp) == EAGLE3_OK && c == 101 && sp == 0);
  CHECK(eagle3_ledger_chain(l, 0, 3, 0, &g) == EAGLE3_OK && g == 0);
  /* speculative rows kept, then a rebuild refused until rewound */
  CHECK(eagle3_ledger_chain(l, 1, 3, EAGLE3_KEEP_SPEC, &g) == EAGLE3_OK && g == 3);
  CHECK(eagle3_ledger_len(l, 1, &c, &sp) == EAGLE3_OK && c == 0 && sp == 3);
  CHECK(eagle3_ledger_chain(l, 1, 3, 0, &g) == EAGLE3_E_STATE);
  CHECK(eagle3_ledger_rewind(l, 1, 1) == EAGLE3_E_INVAL);           /* above committed */
  CHECK(eagle3_ledger_rewind(l, 1, 0) == EAGLE3_OK);
  CHECK(eagle3_ledger_len(l, 1, &c, &sp) == EAGLE3_OK && c == 0 && sp == 0);
  /* bad ids and flags change nothing */
  CHECK(eagle3_ledger_prefill(l, 2, 1, 0) == EAGLE3_E_INVAL);
  CHECK(eagle3_ledger_prefill(l, -1, 1, 0) == EAGLE3_E_INVAL);
  CHECK(eagle3_ledger_chain(l, 0, 3, 64u, &g) == EAGLE3_E_INVAL);
  CHECK(eagle3_ledger_chain(l, 0, 3, EAGLE3_KEEP_SPEC | EAGLE3_ROUND_LOCAL, &g) == EAGLE3_E_INVAL);
  CHECK(eagle3_ledger_chain(l, 0, 3, EAGLE3_STORED_BOUNDARY, &g) == EAGLE3_E_STATE);
  CHECK(eagle3_ledger_len(l, 0, &c, &sp) == EAGLE3_OK && c == 101 && sp == 0);
  CHECK(eagle3_ledger_len(l, 5, &c, &sp) == EAGLE3_E_INVAL);
  eagle3_ledger_destroy(l);
}

static void check_rope(void) {
  int32_t r = -1;
  CHECK(eagle3_resolve_rope_dim(-1, 0.25f, 256, &r) == EAGLE3_OK && r == 64);
  CHECK(eagle3_resolve_rope_dim(32, 0.25f, 256, &r) == EAGLE3_OK && r == 32);
  CHECK(eagle3_resolve_rope_dim(-1, -1.f, 256, &r) == EAGLE3_OK && r == 256);
  CHECK(eagle3_resolve_rope_dim(-1, 2.0f, 256, &r) == EAGLE3_OK && r == 256);
  CHECK(eagle3_resolve_rope_dim(-1, 0.0f, 256, &r) == EAGLE3_OK && r == 256);
  CHECK(eagle3_resolve_rope_dim(-1, NAN, 256, &r) == EAGLE3_OK && r == 256);
  CHECK(eagle3_resolve_rope_dim(33, -1.f, 256, &r) == EAGLE3_E_UNSUPPORTED);
  CHECK(eagle3_resolve_rope_dim(512, -1.f, 256, &r) == EAGLE3_E_UNSUPPORTED);
  CHECK(eagle3_resolve_rope_dim(-1, 0.3f, 64, &r) == EAGLE3_E_UNSUPPORTED);
  CHECK(eagle3_resolve_rope_dim(-1, 0.25f, 256, NULL) == EAGLE3_E_INVAL);
}

/* every check of eagle3_load that fails before device work: the pointers are
   never dereferenced on the device (a dummy non-null address stands in) */
static void check_load_validation(void) {
  eagle3_config c = small_config();
  eagle3_weights w;
  memset(&w, 0, sizeof w);
  const void* dummy = (const void*)(uintptr_t)0x1000;
  const void** f = (const void**)&w.fc;
  for (int i = 0; i < 14; ++i) f[i] = dummy;
  int64_t* d2t = (int64_t*)calloc((size_t)c.draft_vocab, sizeof(int64_t));
  for (int i = 0; i < c.draft_vocab; ++i) d2t[i] = i;  /* target = 2i < 4096 */
  w.d2t_host = d2t;
  w.d2t_len = c.draft_vocab;
  fill_shapes(&c, &w);
  eagle3_ctx* ctx = (eagle3_ctx*)(uintptr_t)1;
  CHECK(eagle3_load(NULL, &w, NULL, &ctx) == EAGLE3_E_INVAL && ctx == NULL);
  CHECK(eagle3_load(&c, &w, NULL, NULL) == EAGLE3_E_INVAL);
  eagle3_config b = c; b.n_aux = 2;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_UNSUPPORTED && ctx == NULL);
  b = c; b.head_dim = 96;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_UNSUPPORTED);
  b = c; b.rope_dim = 63;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_UNSUPPORTED);
  b = c; b.n_head = 5;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_SHAPE);
  b = c; b.kv_dtype = 7;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  b = c; b.append_act = 9;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  b = c; b.token_table = 3;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  b = c; b.token_table = -1;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  b = c; b.kv_dtype = EAGLE3_KV_Q8Q5;  /* batch-1 only */
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_UNSUPPORTED);
  b = c; b.max_ctx = 0;
  CHECK(eagle3_load(&b, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  eagle3_weights v = w; v.embed = NULL;   /* a head without an embedding table */
  CHECK(eagle3_load(&c, &v, NULL, &ctx) == EAGLE3_E_INVAL);
  v = w; v.shape[0][1] = 2 * c.n_embd;    /* fc in != 3n */
  CHECK(eagle3_load(&c, &v, NULL, &ctx) == EAGLE3_E_SHAPE);
  v = w; v.shape[12][0] = 1000;           /* lm_head out != draft vocab */
  CHECK(eagle3_load(&c, &v, NULL, &ctx) == EAGLE3_E_SHAPE);
  v = w; v.d2t_len = 5;
  CHECK(eagle3_load(&c, &v, NULL, &ctx) == EAGLE3_E_SHAPE);
  d2t[17] = 1 << 20;                      /* maps outside the target vocabulary */
  CHECK(eagle3_load(&c, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  d2t[17] = -40;
  CHECK(eagle3_load(&c, &w, NULL, &ctx) == EAGLE3_E_INVAL);
  CHECK(ctx == NULL);
  CHECK(strlen(eagle3_last_error(NULL)) > 0);
  free(d2t);
  /* context-free entry points: argument checks before device work */
  CHECK(eagle3_verify_attention(NULL, dummy, dummy, EAGLE3_KV_F32, 100, 10, 4, 8, 2, 128, (float*)dummy,
                                NULL, 0, NULL) == EAGLE3_E_INVAL);
  CHECK(eagle3_verify_attention((const float*)dummy, dummy, dummy, EAGLE3_KV_F32, 100, 10, 4, 8, 2, 96,
                                (float*)dummy, NULL, 0, NULL) == EAGLE3_E_UNSUPPORTED);
  CHECK(eagle3_verify_attention_noalloc((const float*)dummy, dummy, dummy, EAGLE3_KV_F32, 100, 97, 4, 8, 2,
                                        128, (float*)dummy, NULL) == EAGLE3_E_INVAL);
  CHECK(eagle3_draft_chain(NULL, 1, NULL, NULL, NULL, NULL, NULL, 3, 0, NULL, NULL, NULL, NULL) ==
        EAGLE3_E_INVAL);
  CHECK(eagle3_rewind(NULL, 0, 0) == EAGLE3_E_INVAL);
  CHECK(eagle3_free(NULL) == EAGLE3_OK);
}

static void check_trunk_validation(void) {
  eagle3_trunk_config c;
  memset(&c, 0, sizeof c);
  c.n_embd = 256; c.n_head = 4; c.n_head_kv = 2; c.head_dim = 64; c.n_ff = 768; c.vocab = 4096;
  c.n_layers = 2; c.rope_theta = 1e4f; c.rms_eps = 1e-6f; c.max_ctx = 64; c.max_tokens = 16;
  const void* dummy = (const void*)(uintptr_t)0x1000;
  const void* layers[18];
  for (int i = 0; i < 18; ++i) layers[i] = dummy;
  int64_t shapes[21][2] = {{4096, 256}, {256, 1}, {4096, 256}};
  for (int l = 0; l < 2; ++l) {
    const int64_t s[9][2] = {{256, 1}, {256, 256}, {128, 256}, {128, 256}, {256, 256},
                             {256, 1}, {768, 256}, {768, 256}, {256, 768}};
    memcpy(shapes[3 + 9 * l], s, sizeof s);
  }
  eagle3_trunk_weights w = {dummy, dummy, dummy, layers, &shapes[0][0]};
  eagle3_trunk* t = (eagle3_trunk*)(uintptr_t)1;
  eagle3_trunk_config b = c; b.n_layers = 1;
  CHECK(eagle3_trunk_load(&b, &w, NULL, &t) == EAGLE3_E_UNSUPPORTED && t == NULL);
  b = c; b.max_tokens = 65;
  CHECK(eagle3_trunk_load(&b, &w, NULL, &t) == EAGLE3_E_INVAL);
  shapes[5][0] = 100;   /* layer 0 wk rows */
  CHECK(eagle3_trunk_load(&c, &w, NULL, &t) == EAGLE3_E_SHAPE);
  shapes[5][0] = 128;
  layers[4] = NULL;
  CHECK(eagle3_trunk_load(&c, &w, NULL, &t) == EAGLE3_E_INVAL);
  CHECK(t == NULL);
  CHECK(eagle3_trunk_forward(NULL, 1, NULL, NULL, NULL, NULL, NULL, NULL) == EAGLE3_E_INVAL);
  CHECK(eagle3_generate(NULL, 0, NULL, NULL, 1, 1, 1, NULL, NULL, NULL, NULL) == EAGLE3_E_INVAL);
  CHECK(eagle3_trunk_free(NULL) == EAGLE3_OK);
}

/* ---- device mode: allocation failure at every allocation of a load ---- */
static void* dev_zeros(size_t bytes) {
  void* p = NULL;
  if (hipMalloc(&p, bytes) != hipSuccess) return NULL;
  if (hipMemset(p, 0, bytes) != hipSuccess) return NULL;
  return p;
}

static size_t free_bytes(void) {
  size_t f = 0, t = 0;
  (void)hipDeviceSynchronize();
  (void)hipMemGetInfo(&f, &t);
  return f;
}

static void check_alloc_failures(void) {
  eagle3_config c = small_config();
  const size_t n = 256, big = (size_t)4096 * n * 2;  /* the largest tensor: embed / lm_head bf16 */
  void* buf = dev_zeros(big);
  CHECK(buf != NULL);
  if (!buf) return;
  eagle3_weights w;
  memset(&w, 0, sizeof w);
  const void** f = (const void**)&w.fc;
  for (int i = 0; i < 14; ++i) f[i] = buf;
  int64_t* d2t = (int64_t*)calloc((size_t)c.draft_vocab, sizeof(int64_t));
  w.d2t_host = d2t;
  w.d2t_len = c.draft_vocab;
  fill_shapes(&c, &w);
  {  /* a clean load first: the library's code object is mapped onto the GPU then */
    eagle3_ctx* warm = NULL;
    CHECK(eagle3_load(&c, &w, NULL, &warm) == EAGLE3_OK && warm != NULL);
    if (warm) eagle3_free(warm);
  }
  /* every load that fails must hand back each allocation it made: the library's
     own count of live allocations returns to where it was before the call; both
     the batched bf16 form (token table, step-tiled weights) and the batch-1 int4
     form (quantized weights) */
  eagle3_config ci = c;
  ci.max_seqs = 1;
  ci.weight_format = EAGLE3_WEIGHTS_I4;
  const eagle3_config* forms[2] = {&c, &ci};
  const char* names[2] = {"bf16 batched", "int4"};
  for (int fi = 0; fi < 2; ++fi) {
    int oom = 0;
    const int64_t live0 = eagle3_test_live_allocations();
    const size_t free0 = free_bytes();
    for (int k = 1;; ++k) {
      eagle3_test_fail_allocation(k);
      eagle3_ctx* ctx = (eagle3_ctx*)(uintptr_t)1;
      const int rc = eagle3_load(forms[fi], &w, NULL, &ctx);
      eagle3_test_fail_allocation(0);
      if (rc == EAGLE3_OK) {  /* k is past the last allocation: the load succeeded */
        CHECK(ctx != NULL);
        CHECK(eagle3_test_live_allocations() > live0);
        CHECK(eagle3_free(ctx) == EAGLE3_OK);
        CHECK(eagle3_test_live_allocations() == live0);
        break;
      }
      CHECK(rc == EAGLE3_E_OOM);
      CHECK(ctx == NULL);
      CHECK(eagle3_test_live_allocations() == live0);
      ++oom;
      if (k > 400) { CHECK(!"eagle3_load did not finish within 400 allocations"); break; }
    }
    printf("eagle3_load (%s): %d allocation points failed cleanly; live allocations back to %lld; device "
           "free %zu -> %zu bytes\n", names[fi], oom, (long long)live0, free0, free_bytes());
    CHECK(oom > 10);
  }
  /* the trunk */
  eagle3_trunk_config tc;
  memset(&tc, 0, sizeof tc);
  tc.n_embd = 256; tc.n_head = 4; tc.n_head_kv = 2; tc.head_dim = 64; tc.n_ff = 768; tc.vocab = 4096;
  tc.n_layers = 2; tc.rope_theta = 1e4f; tc.rms_eps = 1e-6f; tc.max_ctx = 64; tc.max_tokens = 16;
  const void* layers[18];
  for (int i = 0; i < 18; ++i) layers[i] = buf;
  int64_t shapes[21][2] = {{4096, 256}, {256, 1}, {4096, 256}};
  for (int l = 0; l < 2; ++l) {
    const int64_t s[9][2] = {{256, 1}, {256, 256}, {128, 256}, {128, 256}, {256, 256},
                             {256, 1}, {768, 256}, {768, 256}, {256, 768}};
    memcpy(shapes[3 + 9 * l], s, sizeof s);
  }
  eagle3_trunk_weights tw = {buf, buf, buf, layers, &shapes[0][0]};
  const int64_t live_t0 = eagle3_test_live_allocations();
  const size_t free_t0 = free_bytes();
  int oom = 0;
  for (int k = 1;; ++k) {
    eagle3_test_fail_allocation(k);
    eagle3_trunk* t = (eagle3_trunk*)(uintptr_t)1;
    const int rc = eagle3_trunk_load(&tc, &tw, NULL, &t);
    eagle3_test_fail_allocation(0);
    if (rc == EAGLE3_OK) {
      CHECK(t != NULL);
      CHECK(eagle3_test_live_allocations() > live_t0);
      CHECK(eagle3_trunk_free(t) == EAGLE3_OK);
      CHECK(eagle3_test_live_allocations() == live_t0);
      break;
    }
    CHECK(rc == EAGLE3_E_OOM);
    CHECK(t == NULL);
    CHECK(eagle3_test_live_allocations() == live_t0);
    ++oom;
    if (k > 400) { CHECK(!"eagle3_trunk_load did not finish within 400 allocations"); break; }
  }
  printf("eagle3_trunk_load: %d allocation points failed cleanly; live allocations back to %lld; device free "
         "%zu -> %zu bytes\n", oom, (long long)live_t0, free_t0, free_bytes());
  CHECK(oom > 10);
  free(d2t);
  (void)hipFree(buf);
}

int main(int argc, char** argv) {
  setvbuf(stdout, NULL, _IONBF, 0);  /* every line reaches the caller */
  const int device = argc > 1 && strcmp(argv[1], "device") == 0;
  check_ledger();
  check_rope();
  check_load_validation();
  check_trunk_validation();
  if (device) check_alloc_failures();
  printf("abi_check %s: %d failed checks\n", device ? "device" : "host", failures);
  /* the leak check now (it ends the process if anything leaked), then leave without
     the GPU runtime's exit-time teardown, which releases its own memory after the
     sanitizer's allocator hooks have seen the runtime unload */
  __lsan_do_leak_check();
  _exit(failures ? 1 : 0);
}
