// The verify side on the GPU (include/eagle3_trunk.h): the synthetic target trunk's
// handle (weights, KV cache, window scratch, host length) and the greedy
// speculative-decoding runner that drives the trunk and the drafter round by round.
//
// Device layout (library-owned): weights as given (bf16 [out][in]); norms fp32;
// per layer K then V caches [n_head_kv][max_ctx][head_dim] fp32 (the verify
// attention's layout); window scratch for max_tokens rows; the runner's round
// buffers: tokens [max_tokens + 1] ([0] = the boundary token, then the drafts),
// per tap stream [max_tokens + 1][n] fp32 (row 0 = the boundary position's taps,
// then the window's), verify ids, and the accept result.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/eagle3.h"
#include "../../include/eagle3_trunk.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_trunk_load_error;

constexpr int kTrunkTensors = 9;  // per layer

}  // namespace

struct eagle3_trunk {
  eagle3_trunk_config cfg{};
  std::vector<void*> allocs;
  std::vector<e3::TrunkLayer> layers;
  e3::TrunkArgs args{};
  int len = 0;
  hipStream_t last_stream = nullptr;
  std::string err;
  // runner buffers
  int32_t *r_tok = nullptr, *r_ids = nullptr, *r_res = nullptr;  // r_res: [a, bonus, status, drafts]
  float* r_taps[3] = {nullptr, nullptr, nullptr};
  int32_t* h_res = nullptr;  // pinned host copy of the accept result
};

namespace {

int t_err(eagle3_trunk* t, int code, const std::string& m) {
  if (t) t->err = m; else g_trunk_load_error = m;
  return code;
}

int t_hip(eagle3_trunk* t, hipError_t e, const char* what) {
  return t_err(t, e == hipErrorOutOfMemory ? EAGLE3_E_OOM : EAGLE3_E_HIP,
               std::string(what) + ": " + hipGetErrorString(e));
}

template <typename T>
int t_alloc(eagle3_trunk* t, T** p, size_t count) {
  void* v = nullptr;
  if (e3::alloc_fault_fires()) return t_hip(t, hipErrorOutOfMemory, "hipMalloc (injected failure)");
  const hipError_t e = hipMalloc(&v, std::max<size_t>(count * sizeof(T), 16));
  if (e != hipSuccess) return t_hip(t, e, "hipMalloc");
  t->allocs.push_back(v);
  e3::note_alloc();
  *p = static_cast<T*>(v);
  return EAGLE3_OK;
}

void t_free_all(eagle3_trunk* t) {
  for (void* p : t->allocs) (void)hipFree(p);
  e3::note_free(t->allocs.size());
  t->allocs.clear();
  if (t->h_res) {
    (void)hipHostFree(t->h_res);
    e3::note_free(1);
  }
  t->h_res = nullptr;
}

}  // namespace

extern "C" {

int eagle3_trunk_load(const eagle3_trunk_config* cfg, const eagle3_trunk_weights* w, void* stream,
                      eagle3_trunk** out) {
  g_trunk_load_error.clear();
  if (!out) return t_err(nullptr, EAGLE3_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!cfg || !w || !w->embed || !w->final_norm || !w->lm_head || !w->layers || !w->shapes)
    return t_err(nullptr, EAGLE3_E_INVAL, "config or weights missing");
  const eagle3_trunk_config& c = *cfg;
  if (c.n_embd <= 0 || c.n_head <= 0 || c.n_head_kv <= 0 || c.n_ff <= 0 || c.vocab <= 0 ||
      c.max_ctx < 1 || c.max_tokens < 1)
    return t_err(nullptr, EAGLE3_E_INVAL, "non-positive dimension");
  if (c.n_layers < 2 || c.n_layers > 64) return t_err(nullptr, EAGLE3_E_UNSUPPORTED, "n_layers must be 2..64");
  if (c.n_head % c.n_head_kv) return t_err(nullptr, EAGLE3_E_SHAPE, "n_head % n_head_kv != 0");
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256)
    return t_err(nullptr, EAGLE3_E_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (c.n_embd % 8 || c.n_ff % 8) return t_err(nullptr, EAGLE3_E_UNSUPPORTED, "n_embd and n_ff must be multiples of 8");
  if (!(c.rope_theta > 0.f) || !std::isfinite(c.rope_theta) || !(c.rms_eps >= 0.f))
    return t_err(nullptr, EAGLE3_E_INVAL, "bad rope_theta or rms_eps");
  if (int64_t(c.max_tokens) > c.max_ctx) return t_err(nullptr, EAGLE3_E_INVAL, "max_tokens above max_ctx");
  const int64_t n = c.n_embd, qd = int64_t(c.n_head) * c.head_dim, kvd = int64_t(c.n_head_kv) * c.head_dim,
                ff = c.n_ff, V = c.vocab;
  // declared shapes: embed, final_norm, lm_head, then 9 per layer
  const int64_t per[kTrunkTensors][2] = {{n, 1}, {qd, n}, {kvd, n}, {kvd, n}, {n, qd},
                                         {n, 1}, {ff, n}, {ff, n}, {n, ff}};
  const int count = 3 + kTrunkTensors * c.n_layers;
  for (int i = 0; i < count; ++i) {
    int64_t want[2];
    if (i == 0 || i == 2) { want[0] = V; want[1] = n; }
    else if (i == 1) { want[0] = n; want[1] = 1; }
    else { want[0] = per[(i - 3) % kTrunkTensors][0]; want[1] = per[(i - 3) % kTrunkTensors][1]; }
    if (w->shapes[2 * i] != want[0] || w->shapes[2 * i + 1] != want[1]) {
      char buf[128];
      snprintf(buf, sizeof buf, "tensor %d: declared [%lld, %lld], config implies [%lld, %lld]", i,
               (long long)w->shapes[2 * i], (long long)w->shapes[2 * i + 1], (long long)want[0],
               (long long)want[1]);
      return t_err(nullptr, EAGLE3_E_SHAPE, buf);
    }
    if (i >= 3 && !w->layers[i - 3]) return t_err(nullptr, EAGLE3_E_INVAL, "layer tensor is NULL");
  }
  // verify-attention partials: the most any window may need (the split count
  // depends on the rows attended, so every total is tried)
  size_t ws = 0;
  for (int64_t T = 1; T <= c.max_ctx; ++T) {
    const int M = int(std::min<int64_t>(c.max_tokens, T));
    ws = std::max(ws, e3::attn_verify_workspace(M, c.n_head, c.n_head_kv, c.head_dim, int(T - M), 1));
  }

  eagle3_trunk* t = new (std::nothrow) eagle3_trunk();
  if (!t) return t_err(nullptr, EAGLE3_E_OOM, "host allocation failed");
  t->cfg = c;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto fail = [&](int code) {
    g_trunk_load_error = t->err;
    (void)hipDeviceSynchronize();
    t_free_all(t);
    delete t;
    return code;
  };
#define T_TRY(x)              \
  do {                        \
    int _rc = (x);            \
    if (_rc) return fail(_rc); \
  } while (0)
#define T_HIP(x, what)                                    \
  do {                                                    \
    hipError_t _e = (x);                                  \
    if (_e != hipSuccess) return fail(t_hip(t, _e, what)); \
  } while (0)
  auto copy_bf16 = [&](uint16_t** dst, const void* src, size_t count) -> int {
    int rc = t_alloc(t, dst, count);
    if (rc) return rc;
    const hipError_t e = hipMemcpyAsync(*dst, src, count * 2, hipMemcpyDeviceToDevice, s);
    return e == hipSuccess ? EAGLE3_OK : t_hip(t, e, "copy weights");
  };
  auto copy_norm = [&](float** dst, const void* src) -> int {
    int rc = t_alloc(t, dst, size_t(n));
    if (rc) return rc;
    const hipError_t e = e3::launch_bf16_to_f32(static_cast<const uint16_t*>(src), *dst, int(n), s);
    return e == hipSuccess ? EAGLE3_OK : t_hip(t, e, "convert norm");
  };
  e3::TrunkArgs& a = t->args;
  a.n = int(n); a.nh = c.n_head; a.nkv = c.n_head_kv; a.hd = c.head_dim; a.ff = int(ff);
  a.vocab = int(V); a.n_layers = c.n_layers; a.cap = c.max_ctx; a.eps = c.rms_eps;
  uint16_t *embed = nullptr, *lm = nullptr;
  float* fnorm = nullptr;
  T_TRY(copy_bf16(&embed, w->embed, size_t(V * n)));
  T_TRY(copy_bf16(&lm, w->lm_head, size_t(V * n)));
  T_TRY(copy_norm(&fnorm, w->final_norm));
  a.embed = embed; a.lm_head = lm; a.final_norm = fnorm;
  t->layers.resize(size_t(c.n_layers));
  for (int l = 0; l < c.n_layers; ++l) {
    const void* const* src = w->layers + size_t(l) * kTrunkTensors;
    e3::TrunkLayer& L = t->layers[size_t(l)];
    float *an = nullptr, *mn = nullptr;
    uint16_t* m[7] = {};
    T_TRY(copy_norm(&an, src[0]));
    T_TRY(copy_bf16(&m[0], src[1], size_t(qd * n)));
    T_TRY(copy_bf16(&m[1], src[2], size_t(kvd * n)));
    T_TRY(copy_bf16(&m[2], src[3], size_t(kvd * n)));
    T_TRY(copy_bf16(&m[3], src[4], size_t(n * qd)));
    T_TRY(copy_norm(&mn, src[5]));
    T_TRY(copy_bf16(&m[4], src[6], size_t(ff * n)));
    T_TRY(copy_bf16(&m[5], src[7], size_t(ff * n)));
    T_TRY(copy_bf16(&m[6], src[8], size_t(n * ff)));
    L.attn_norm = an; L.mlp_norm = mn;
    L.wq = m[0]; L.wk = m[1]; L.wv = m[2]; L.wo = m[3]; L.w_gate = m[4]; L.w_up = m[5]; L.w_down = m[6];
    T_TRY(t_alloc(t, &L.k_cache, size_t(kvd) * c.max_ctx));
    T_TRY(t_alloc(t, &L.v_cache, size_t(kvd) * c.max_ctx));
  }
  a.layer = t->layers.data();
  double* invf_d = nullptr;
  T_TRY(t_alloc(t, &invf_d, size_t(c.head_dim / 2)));
  std::vector<double> invf(size_t(c.head_dim / 2));
  for (int i = 0; i < c.head_dim / 2; ++i)
    invf[size_t(i)] = std::pow(double(c.rope_theta), -2.0 * double(i) / double(c.head_dim));
  T_HIP(hipMemcpyAsync(invf_d, invf.data(), invf.size() * sizeof(double), hipMemcpyHostToDevice, s),
        "copy inv_freq");
  a.inv_freq = invf_d;
  const size_t R = size_t(c.max_tokens);
  e3::TrunkBufs& b = a.buf;
  T_TRY(t_alloc(t, &b.x, R * n));
  T_TRY(t_alloc(t, &b.h, R * n));
  T_TRY(t_alloc(t, &b.z, R * n));
  T_TRY(t_alloc(t, &b.q, R * qd));
  T_TRY(t_alloc(t, &b.k, R * kvd));
  T_TRY(t_alloc(t, &b.v, R * kvd));
  T_TRY(t_alloc(t, &b.o, R * qd));
  T_TRY(t_alloc(t, &b.act, R * ff));
  T_TRY(t_alloc(t, &b.logits, R * V));
  b.ws_bytes = ws;
  T_TRY(t_alloc(t, &b.part_o, ws / sizeof(float) + 4));
  b.part_ml = b.part_o + ws / sizeof(float) / size_t(c.head_dim + 2) * size_t(c.head_dim);
  T_TRY(t_alloc(t, &a.status, 1));
  T_HIP(hipMemsetAsync(a.status, 0, 4, s), "clear status");
  T_TRY(t_alloc(t, &t->r_tok, R + 1));
  T_TRY(t_alloc(t, &t->r_ids, R));
  T_TRY(t_alloc(t, &t->r_res, R + 3));
  for (int j = 0; j < 3; ++j) T_TRY(t_alloc(t, &t->r_taps[j], (R + 1) * n));
  if (e3::alloc_fault_fires()) return fail(t_hip(t, hipErrorOutOfMemory, "hipHostMalloc (injected failure)"));
  T_HIP(hipHostMalloc(reinterpret_cast<void**>(&t->h_res), (R + 3) * sizeof(int32_t)), "pinned result");
  e3::note_alloc();
  T_HIP(hipStreamSynchronize(s), "load sync");
#undef T_TRY
#undef T_HIP
  *out = t;
  return EAGLE3_OK;
}

int eagle3_trunk_free(eagle3_trunk* t) {
  if (!t) return EAGLE3_OK;
  (void)hipDeviceSynchronize();
  t_free_all(t);
  delete t;
  return EAGLE3_OK;
}

const char* eagle3_trunk_last_error(const eagle3_trunk* t) {
  return t ? t->err.c_str() : g_trunk_load_error.c_str();
}

int eagle3_trunk_forward(eagle3_trunk* t, int32_t T, const int32_t* tok_dev, int32_t* ids_dev,
                         float* tap0_dev, float* tap1_dev, float* tap2_dev, void* stream) {
  if (!t) return EAGLE3_E_INVAL;
  if (!tok_dev || !ids_dev) return t_err(t, EAGLE3_E_INVAL, "null token or id pointer");
  if (T < 1 || T > t->cfg.max_tokens) return t_err(t, EAGLE3_E_INVAL, "window size outside 1..max_tokens");
  if (int64_t(t->len) + T > t->cfg.max_ctx) return t_err(t, EAGLE3_E_CAPACITY, "trunk KV capacity exceeded");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* const taps[3] = {tap0_dev, tap1_dev, tap2_dev};
  const hipError_t e = e3::launch_trunk_forward(t->args, T, t->len, tok_dev, ids_dev, taps, s);
  if (e != hipSuccess) return t_hip(t, e, "trunk forward");
  t->len += T;
  t->last_stream = s;
  return EAGLE3_OK;
}

int eagle3_trunk_rollback(eagle3_trunk* t, int32_t new_len) {
  if (!t) return EAGLE3_E_INVAL;
  if (new_len < 0 || new_len > t->len) return t_err(t, EAGLE3_E_INVAL, "rollback beyond the cache length");
  t->len = new_len;
  return EAGLE3_OK;
}

int eagle3_trunk_len(const eagle3_trunk* t, int32_t* len) {
  if (!t || !len) return EAGLE3_E_INVAL;
  *len = t->len;
  return EAGLE3_OK;
}

int eagle3_trunk_status(eagle3_trunk* t, uint32_t* flags) {
  if (!t || !flags) return EAGLE3_E_INVAL;
  hipError_t e = hipStreamSynchronize(t->last_stream);
  uint32_t v = 0;
  if (e == hipSuccess) e = hipMemcpy(&v, t->args.status, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(t->args.status, 0, 4);
  if (e != hipSuccess) return t_hip(t, e, "trunk status");
  *flags = v;
  return EAGLE3_OK;
}

int eagle3_generate(eagle3_ctx* dr, int32_t seq, eagle3_trunk* t, const int32_t* prompt_host,
                    int32_t prompt_len, int32_t max_new, int32_t gamma, int32_t* out_host,
                    int64_t* drafted, int64_t* accepted, void* stream) {
  if (!t) return EAGLE3_E_INVAL;
  if (!dr || !prompt_host || !out_host) return t_err(t, EAGLE3_E_INVAL, "null argument");
  if (prompt_len < 1 || prompt_len > t->cfg.max_tokens)
    return t_err(t, EAGLE3_E_INVAL, "prompt length outside 1..max_tokens");
  if (max_new < 1 || gamma < 1 || gamma + 1 > t->cfg.max_tokens)
    return t_err(t, EAGLE3_E_INVAL, "max_new or gamma out of range");
  if (int64_t(prompt_len) + max_new + gamma > t->cfg.max_ctx)
    return t_err(t, EAGLE3_E_CAPACITY, "trunk KV too small for prompt + max_new + gamma");
  int32_t committed = 0, spec = 0;
  int rc = eagle3_kv_len(dr, seq, &committed, &spec);
  if (rc) return t_err(t, rc, "bad drafter sequence");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t n = size_t(t->cfg.n_embd);
  auto drafter_fail = [&](int code, const char* what) {
    return t_err(t, code, std::string(what) + ": " + eagle3_last_error(dr));
  };
  auto hip_ok = [&](hipError_t e, const char* what) { return e == hipSuccess ? EAGLE3_OK : t_hip(t, e, what); };
  auto status_error = [&](uint32_t f) -> int {
    if (f & EAGLE3_TRUNK_BAD_TOKEN) return t_err(t, EAGLE3_E_INVAL, "trunk: an id outside the vocabulary");
    if (f & EAGLE3_TRUNK_NAN_LOGITS) return t_err(t, EAGLE3_E_HIP, "trunk: logits are all NaN");
    return EAGLE3_OK;
  };
  auto check_status = [&]() -> int {
    uint32_t f = 0;
    if (int r = eagle3_trunk_status(t, &f)) return r;
    return status_error(f);
  };
  float* taps[3] = {t->r_taps[0], t->r_taps[1], t->r_taps[2]};
  auto tap_rows = [&](int row) {
    return std::vector<float*>{taps[0] + size_t(row) * n, taps[1] + size_t(row) * n, taps[2] + size_t(row) * n};
  };
  t->len = 0;
  if ((rc = eagle3_rewind(dr, seq, 0))) return drafter_fail(rc, "rewind");

  // prompt: the trunk's taps of every prompt position and x_P
  const int P = prompt_len;
  if ((rc = hip_ok(hipMemcpyAsync(t->r_tok, prompt_host, size_t(P) * 4, hipMemcpyHostToDevice, s), "prompt")))
    return rc;
  if ((rc = eagle3_trunk_forward(t, P, t->r_tok, t->r_ids, taps[0], taps[1], taps[2], stream))) return rc;
  // drafter rows (taps of r, x_{r+1}), r < P - 1; the boundary feature from the taps of P - 1
  {
    std::vector<float*> bnd = tap_rows(P - 1);
    rc = eagle3_prefill(dr, seq, P - 1, P > 1 ? t->r_tok + 1 : nullptr, P > 1 ? taps[0] : nullptr,
                        P > 1 ? taps[1] : nullptr, P > 1 ? taps[2] : nullptr, bnd[0], bnd[1], bnd[2], stream);
    if (rc) return drafter_fail(rc, "prefill");
  }
  // round buffers: tokens [boundary, drafts...]; taps row 0 = the boundary position's
  for (int j = 0; j < 3; ++j)
    if ((rc = hip_ok(hipMemcpyAsync(taps[j], taps[j] + size_t(P - 1) * n, n * 4, hipMemcpyDeviceToDevice, s),
                     "boundary taps")))
      return rc;
  if ((rc = hip_ok(hipMemcpyAsync(t->r_tok, t->r_ids + (P - 1), 4, hipMemcpyDeviceToDevice, s), "x_P")))
    return rc;
  if ((rc = hip_ok(hipMemcpyAsync(t->h_res, t->r_ids + (P - 1), 4, hipMemcpyDeviceToHost, s), "x_P")))
    return rc;
  if ((rc = hip_ok(hipStreamSynchronize(s), "sync"))) return rc;
  if ((rc = check_status())) return rc;
  int emitted = 0;
  out_host[emitted++] = t->h_res[0];
  int64_t n_drafted = 0, n_accepted = 0;
  int pos = P;  // position of the boundary token
  while (emitted < max_new) {
    int32_t geff = 0;
    rc = eagle3_draft_chain(dr, 1, &seq, t->r_tok, nullptr, nullptr, nullptr, gamma, EAGLE3_STORED_BOUNDARY,
                            t->r_tok + 1, &geff, nullptr, stream);
    if (rc) return drafter_fail(rc, "draft_chain");
    // the verify window [x_n, d_1 .. d_geff]: its taps into rows 1 .. geff + 1
    std::vector<float*> win = tap_rows(1);
    if ((rc = eagle3_trunk_forward(t, geff + 1, t->r_tok, t->r_ids, win[0], win[1], win[2], stream))) return rc;
    if ((rc = hip_ok(e3::launch_accept(t->r_tok + 1, t->r_ids, geff, t->r_res, t->args.status, s), "accept")))
      return rc;
    if ((rc = hip_ok(hipMemcpyAsync(t->h_res, t->r_res, size_t(geff + 3) * 4, hipMemcpyDeviceToHost, s),
                     "accept result")))
      return rc;
    if ((rc = hip_ok(hipStreamSynchronize(s), "sync"))) return rc;
    if ((rc = status_error(uint32_t(t->h_res[2])))) return rc;
    const int a = t->h_res[0], bonus = t->h_res[1];
    if (a < 0 || a > geff) return t_err(t, EAGLE3_E_HIP, "accept walk out of range");
    n_drafted += geff;
    n_accepted += a;
    for (int i = 0; i < a && emitted < max_new; ++i) out_host[emitted++] = t->h_res[3 + i];
    if (emitted < max_new) out_host[emitted++] = bonus;
    if ((rc = eagle3_trunk_rollback(t, pos + a + 1))) return rc;
    // commit (taps of n - 1, x_n), (taps of n + i - 1, d_i) for i <= a; the next
    // boundary feature from the taps of n + a (window row a + 1)
    std::vector<float*> nb = tap_rows(a + 1);
    rc = eagle3_rebuild_after_verify(dr, 1, &seq, &a, t->r_tok, taps[0], taps[1], taps[2], nb[0], nb[1], nb[2],
                                     stream);
    if (rc) return drafter_fail(rc, "rebuild_after_verify");
    for (int j = 0; j < 3; ++j)
      if ((rc = hip_ok(hipMemcpyAsync(taps[j], nb[size_t(j)], n * 4, hipMemcpyDeviceToDevice, s), "next taps")))
        return rc;
    if ((rc = hip_ok(hipMemcpyAsync(t->r_tok, t->r_res + 1, 4, hipMemcpyDeviceToDevice, s), "bonus"))) return rc;
    pos += a + 1;
  }
  if ((rc = hip_ok(hipStreamSynchronize(s), "sync"))) return rc;
  if (drafted) *drafted = n_drafted;
  if (accepted) *accepted = n_accepted;
  return EAGLE3_OK;
}

}  // extern "C"
