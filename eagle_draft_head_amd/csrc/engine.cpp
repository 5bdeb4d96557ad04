// eagle3 engine: the C ABI of include/eagle3.h on top of the gfx950 kernels.
//
// Device layout (all library-owned):
//   weights  fc [n, 3n]; qkv [(nh + 2 nkv) hd, 2n] with the q and k rows of every
//            head reordered so that rotary partners (i, i + rope_dim/2) are
//            adjacent rows; o [n, nh hd]; gate/up interleaved [2 ff, n]
//            (row 2i = gate_i, 2i+1 = up_i); down [n, ff]; lm_head [dv, n];
//            embedding [Vt, n]; the four norm vectors as fp32; d2t as int32.
//   draft KV per sequence: K [nkv][max_ctx + 1][hd] then V, fp32 (or bf16), head-major
//            so one KV head's rows are contiguous for the attention stream.
//   chain scratch (fp32 vectors, split-attention partials, argmax partials,
//            device token slots).
//   append scratch for up to `tf_rows` teacher-forced rows per GEMM pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/eagle3.h"
#include "../../include/eagle3_ledger.h"
#include "../../include/eagle3_testing.h"
#include "gemv_cfg.hpp"
#include "kernels.hpp"
#include "ledger.hpp"

namespace e3 {

namespace {
std::atomic<int32_t> g_alloc_fault{0};
std::atomic<int64_t> g_live_allocs{0};
}  // namespace

void note_alloc() { g_live_allocs.fetch_add(1, std::memory_order_relaxed); }
void note_free(size_t n) { g_live_allocs.fetch_sub(int64_t(n), std::memory_order_relaxed); }

bool alloc_fault_fires() {
  int32_t v = g_alloc_fault.load(std::memory_order_relaxed);
  while (v > 0) {
    if (g_alloc_fault.compare_exchange_weak(v, v - 1, std::memory_order_relaxed)) return v == 1;
  }
  return false;
}

}  // namespace e3

namespace {

thread_local std::string g_load_error;

constexpr int kProfKernels = 10;
// gfx950 gives a workgroup up to 160 KB of LDS; the GEMVs keep one fp32
// activation vector there (the down projection of a 5120-wide drafter: 68 KB)
constexpr int64_t kMaxStageBytes = 128 * 1024;
constexpr int64_t kMaxLdsBytes = 160 * 1024;  // a workgroup's LDS on gfx950

struct Profiler {
  int kernel = -1;
  std::vector<hipEvent_t> ev;  // pairs
  size_t used = 0;
};

}  // namespace

struct eagle3_ctx {
  eagle3_config cfg{};
  int device = 0;
  int n = 0, nh = 0, nkv = 0, hd = 0, qd = 0, kvd = 0, ff = 0, dv = 0, vt = 0, rot = 0, cap = 0;
  std::vector<void*> allocs;

  // int4 projection weights (weight_format EAGLE3_WEIGHTS_I4): codes and scales of
  // each matrix, rows in the same (repacked) order as the bf16 copies
  struct I4W {
    uint8_t* q = nullptr;
    uint16_t* s = nullptr;
  } i4_fc, i4_qkv, i4_o, i4_gu, i4_d, i4_lm;
  bool i4 = false;
  // int4: the teacher-forced MFMA passes multiply by the int4 weights of fc and of the
  // K/V rows of QKV as exact bf16 (hi, lo) pairs: hi overwrites those rows of w_fc /
  // w_qkv, lo lives here
  uint16_t *i4_fc_lo = nullptr, *i4_qkv_lo = nullptr, *i4_kv_lo = nullptr;  // kv: rows qd.. of qkv
  // the weight stream a GEMV reads: the bf16 rows or the int4 codes, and the scales
  const uint16_t* wq(const uint16_t* bf16, const I4W& m, size_t row0 = 0, size_t K = 0) const {
    return i4 ? reinterpret_cast<const uint16_t*>(m.q + row0 * (K / 2)) : bf16 + row0 * K;
  }
  const uint16_t* ws(const I4W& m, size_t row0 = 0, size_t K = 0) const {
    return i4 ? m.s + row0 * (K / 32) : nullptr;
  }
  uint16_t *w_fc = nullptr, *w_qkv = nullptr, *w_o = nullptr, *w_gu = nullptr, *w_d = nullptr,
           *w_lm = nullptr, *embed = nullptr;
  float *nrm_in = nullptr, *nrm_hid = nullptr, *nrm_post = nullptr, *nrm_fin = nullptr;
  int32_t* d2t = nullptr;
  uint32_t* status = nullptr;  // device status word (e3::kStatus* bits)
  double* inv_freq = nullptr;  // [rot / 2]
  int gcfg[e3::kGemvKinds] = {};
  int lm_grid = 0;
  char* kv = nullptr;
  int kv_f32 = 1;
  int kv_q = 0;             // quantized K/V regions (q8_0 K, q5_1 V); elements are bytes
  int tf_split = 0;         // teacher-forced MFMA passes take (hi, lo) bf16 activation pairs
  int tf_f16 = 0;           // ... or one fp16 term against fp16 weight copies scaled by 2^8
  uint16_t *w_fc16 = nullptr, *w_kv16 = nullptr;  // tf_f16: fc and the K/V rows of QKV, fp16 x 2^8
  float* kv_stage = nullptr;  // kv_q: the chain step's new K/V row in fp32 [2][kvd]
  size_t kv_esize = 4;      // bytes per cache element
  size_t kv_seq_elems = 0;  // K + V elements per sequence

  // recurrent hidden buffers: [0] the encoded boundary feature, [1]/[2] g_next of
  // alternating steps; each with its hidden_norm- and norm-weighted copies and
  // the per-block partial sums of its squares
  struct GBuf {
    float *y = nullptr, *w_hid = nullptr, *w_norm = nullptr, *ssq = nullptr;
    int count = 0;
  } gb[3];
  float *x1 = nullptr, *x1w = nullptr, *x1_ssq = nullptr, *act = nullptr, *q = nullptr,
        *ao = nullptr, *part_o = nullptr, *part_ml = nullptr, *lm_pv = nullptr;
  int x1_count = 0;
  int32_t *lm_pi = nullptr, *lm_pt = nullptr, *tok_slots = nullptr;
  // stored boundary features per sequence slot (set by prefill / rebuild when the
  // next round's boundary taps come with them): f [max_seqs][n], f * hidden_norm
  // [max_seqs][n] and sum f^2 [max_seqs]
  float *bnd_y = nullptr, *bnd_w = nullptr, *bnd_ssq = nullptr;
  // round-local scratch KV (EAGLE3_ROUND_LOCAL): per slot K then V, each
  // [n_head_kv][max_gamma][head_dim]
  char* kv_local = nullptr;
  int cap_local = 0;
  size_t kv_local_elems = 0;  // K + V elements per slot

  // token table of the chain step's QKV embedding half: [target_vocab][N_qkv] fp32
  // rows of W_qkv[:, :n] . (input_layernorm * E[t]) / rms(E[t]) in the repacked row
  // order, and sum E[t]^2 per token, which the build uses (null when off)
  float *tok_tab = nullptr, *tok_ss = nullptr;
  // deferred QKV of the batch-1 chain step (with the token table and bf16 weights):
  // the hidden half of every QKV row, computed in the previous step's lm_head launch
  // (or alone for a chain's first step) and finished by the attention kernel
  float* hsum = nullptr;
  bool defer_qkv = false;
  // with the deferred QKV: the hidden-half sums of each slot's stored
  // boundary feature [max_seqs][N_qkv], computed by the append pass that writes the
  // feature (its K/V launch); bnd_hsum_ok[slot] says whether the slot's current
  // feature came with them (EAGLE3_BOUNDARY_QH=0: never, for comparison)
  float* bnd_hsum = nullptr;
  std::vector<uint8_t> bnd_hsum_ok;
  // with the table (bf16 weights): the hidden half of W_qkv as a contiguous [N][n]
  // matrix, the only part of W_qkv a chain step streams
  uint16_t* w_qkv_h = nullptr;
  const uint16_t* hid_rows() const { return w_qkv_h ? w_qkv_h : w_qkv + n; }
  size_t hid_ldw() const { return w_qkv_h ? size_t(n) : size_t(2) * n; }
  // the deferred QKV's hidden-half stream of g: bf16 rows, or the int4 codes of
  // columns n .. 2n of W_qkv
  e3::QhArgs qh_args(const GBuf& g) const {
    const int N = (nh + 2 * nkv) * hd;
    if (i4)
      return e3::QhArgs{reinterpret_cast<const uint16_t*>(i4_qkv.q), i4_qkv.s, size_t(2) * n, n, N, n, g.w_hid,
                        g.ssq, g.count, cfg.rms_eps, hsum};
    return e3::QhArgs{hid_rows(), nullptr, hid_ldw(), 0, N, n, g.w_hid, g.ssq, g.count, cfg.rms_eps, hsum};
  }

  int tf_rows = 0;
  size_t tf_F_cap = 0, tf_P_cap = 0;  // floats
  uint16_t *tf_A = nullptr, *tf_A_lo = nullptr, *tf_cat16 = nullptr, *tf_cat16_lo = nullptr;
  float *tf_cat32 = nullptr, *tf_F = nullptr, *tf_P = nullptr;

  // batched drafting scratch (max_seqs > 1): activation pairs A (fc input, cat,
  // normed x1 / g_next) and B (attention output, SiLU product), split-K partials,
  // per-row vectors, attention partials, lm_head candidates
  int bld_a = 0, bld_b = 0;
  uint16_t *bx_a_hi = nullptr, *bx_a_lo = nullptr, *bx_b_hi = nullptr, *bx_b_lo = nullptr;
  float *b_P = nullptr, *b_G = nullptr, *b_X1 = nullptr, *b_q = nullptr, *b_po = nullptr,
        *b_pml = nullptr, *b_cand_v = nullptr, *b_logits = nullptr;
  // normalised inputs of the gate/up and lm_head GEMMs as (hi, lo) pairs [32][n]
  uint16_t *bx_z_hi = nullptr, *bx_z_lo = nullptr, *bx_h_hi = nullptr, *bx_h_lo = nullptr;
  int32_t* b_cand_i = nullptr;
  e3::BGemmPlan bp_enc{}, bp_qkv{}, bp_o{}, bp_gu{}, bp_d{}, bp_lm{};
  // LDS-tiled plans of the same projections (splits 0: K is not a multiple of 64,
  // the fragment-load GEMM above runs instead)
  e3::GemmPlan tp_enc{}, tp_qkv{}, tp_o{}, tp_gu{}, tp_d{}, tp_lm{};
  // step-tiled copies of the projections those plans stream (e3::launch_tile_weights;
  // null where the plan is the fragment-load GEMM)
  uint16_t *bt_enc = nullptr, *bt_qkv = nullptr, *bt_o = nullptr, *bt_gu = nullptr, *bt_d = nullptr,
           *bt_lm = nullptr;
  int b_ncand = 0;  // lm_head candidates per batch row

  e3::Ledger ledger;
  std::string err;
  Profiler prof;

  void* k_of(int s) { return kv + size_t(s) * kv_seq_elems * kv_esize; }
  void* k_local(int s) { return kv_local + size_t(s) * kv_local_elems * kv_esize; }
  void* v_local(int s) { return kv_local + (size_t(s) * kv_local_elems + kv_local_elems / 2) * kv_esize; }
  void* v_of(int s) { return kv + (size_t(s) * kv_seq_elems + kv_seq_elems / 2) * kv_esize; }
};

struct eagle3_ledger {
  e3::Ledger l;
};

namespace {

int set_err(eagle3_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg; else g_load_error = msg;
  return code;
}

int hip_fail(eagle3_ctx* c, hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return set_err(c, e == hipErrorOutOfMemory ? EAGLE3_E_OOM : EAGLE3_E_HIP, m);
}

// Launch-configuration override of the batch-1 GEMV kernels, for tuning on new
// shapes: EAGLE3_GEMV_CONFIG="qkv=8,o=5,..." (kinds encode, qkv, o, gateup,
// down, lmhead; ids index E3_GEMV_CONFIGS).  The fused qkv and gate/up kernels
// need an even row count per wave.
int gemv_config_override(eagle3_ctx* c) {
  const char* env = std::getenv("EAGLE3_GEMV_CONFIG");
  if (!env || !*env) return EAGLE3_OK;
  static const char* names[e3::kGemvKinds] = {"encode", "qkv", "o", "gateup", "down", "lmhead"};
  std::string spec(env);
  size_t at = 0;
  while (at < spec.size()) {
    size_t end = spec.find(',', at);
    if (end == std::string::npos) end = spec.size();
    const std::string item = spec.substr(at, end - at);
    at = end + 1;
    const size_t eq = item.find('=');
    int kind = -1;
    for (int k = 0; k < e3::kGemvKinds && eq != std::string::npos; ++k)
      if (item.compare(0, eq, names[k]) == 0 && std::strlen(names[k]) == eq) kind = k;
    char* tail = nullptr;
    const long id = eq == std::string::npos ? -1 : std::strtol(item.c_str() + eq + 1, &tail, 10);
    const int rows = (id >= 0 && id < e3::kGemvConfigCount) ? e3::gemv_cfg_rows(int(id)) : -1;
    const bool paired = kind == e3::kGemvQkv || kind == e3::kGemvGateUp;
    if (kind < 0 || rows < 0 || (tail && *tail) || (paired && rows % 2))
      return set_err(c, EAGLE3_E_INVAL, "EAGLE3_GEMV_CONFIG: bad item '" + item + "'");
    c->gcfg[kind] = int(id);
  }
  return EAGLE3_OK;
}

#define E3_HIP(ctx, expr, what)                    \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(ctx, _e, what); \
  } while (0)

template <typename T>
int dalloc(eagle3_ctx* c, T** p, size_t count) {
  void* v = nullptr;
  if (e3::alloc_fault_fires()) return hip_fail(c, hipErrorOutOfMemory, "hipMalloc (injected failure)");
  hipError_t e = hipMalloc(&v, count * sizeof(T) > 0 ? count * sizeof(T) : 16);
  if (e != hipSuccess) return hip_fail(c, e, "hipMalloc");
  c->allocs.push_back(v);
  e3::note_alloc();
  *p = static_cast<T*>(v);
  return EAGLE3_OK;
}

void free_all(eagle3_ctx* c) {
  for (void* p : c->allocs) (void)hipFree(p);
  e3::note_free(c->allocs.size());
  c->allocs.clear();
  for (hipEvent_t e : c->prof.ev) (void)hipEventDestroy(e);
  c->prof.ev.clear();
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// activation inputs are read in 16-byte vectors
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// --- profiling of one kernel family with events on the launching stream -----
// A scope of one kernel launch (one_launch) hands its event pair to that launch,
// which records the kernel's own start and end (hipExtLaunchKernelGGL); a scope of
// several launches records the pair around them on the stream.
struct ProfScope {
  eagle3_ctx* c;
  hipStream_t s;
  bool on, single;
  ProfScope(eagle3_ctx* cx, int kernel, hipStream_t st, bool one_launch = false)
      : c(cx), s(st), on(false), single(one_launch) {
    if (c->prof.kernel == kernel && c->prof.used + 2 <= c->prof.ev.size()) {
      on = true;
      if (single) {
        e3::g_launch_ev.start = c->prof.ev[c->prof.used];
        e3::g_launch_ev.stop = c->prof.ev[c->prof.used + 1];
        e3::g_launch_ev.armed = true;
      } else {
        (void)hipEventRecord(c->prof.ev[c->prof.used], s);
      }
    }
  }
  ~ProfScope() {
    if (on) {
      if (single) e3::g_launch_ev.armed = false;
      else (void)hipEventRecord(c->prof.ev[c->prof.used + 1], s);
      c->prof.used += 2;
    }
  }
};

int validate_config(const eagle3_config* cfg, const char** why) {
  auto bad = [&](const char* m, int code) { *why = m; return code; };
  if (cfg->n_aux != 3) return bad("n_aux must be 3", EAGLE3_E_UNSUPPORTED);
  if (cfg->n_embd <= 0 || cfg->n_head <= 0 || cfg->n_head_kv <= 0 || cfg->head_dim <= 0 ||
      cfg->n_ff <= 0 || cfg->draft_vocab <= 0 || cfg->target_vocab <= 0)
    return bad("non-positive dimension", EAGLE3_E_INVAL);
  if (cfg->max_ctx < 1 || cfg->max_gamma < 1 || cfg->max_seqs < 1)
    return bad("max_ctx, max_gamma and max_seqs must be >= 1", EAGLE3_E_INVAL);
  if (cfg->n_head % cfg->n_head_kv) return bad("n_head % n_head_kv != 0", EAGLE3_E_SHAPE);
  if (cfg->n_head / cfg->n_head_kv > 8) return bad("more than 8 query heads per KV head", EAGLE3_E_UNSUPPORTED);
  if (cfg->head_dim != 64 && cfg->head_dim != 128 && cfg->head_dim != 256)
    return bad("head_dim must be 64, 128 or 256", EAGLE3_E_UNSUPPORTED);
  if (cfg->rope_dim <= 0 || cfg->rope_dim > cfg->head_dim || (cfg->rope_dim & 1))
    return bad("rope_dim must be even and in (0, head_dim]", EAGLE3_E_UNSUPPORTED);
  if (cfg->n_embd % 64) return bad("n_embd must be a multiple of 64", EAGLE3_E_UNSUPPORTED);
  if (cfg->max_seqs > 1 && cfg->n_embd > e3::kBRowMax)
    return bad("batched drafting supports n_embd up to 8192", EAGLE3_E_UNSUPPORTED);
  if (cfg->n_ff % 8) return bad("n_ff must be a multiple of 8", EAGLE3_E_UNSUPPORTED);
  if (!(cfg->rope_theta > 0.f) || !std::isfinite(cfg->rope_theta)) return bad("rope_theta must be > 0", EAGLE3_E_INVAL);
  if (!(cfg->rms_eps >= 0.f) || !std::isfinite(cfg->rms_eps)) return bad("rms_eps must be >= 0", EAGLE3_E_INVAL);
  if (int64_t(cfg->max_ctx) + 1 > (int64_t(1) << 30)) return bad("max_ctx too large", EAGLE3_E_UNSUPPORTED);
  if (cfg->max_gamma > 64) return bad("max_gamma above 64", EAGLE3_E_UNSUPPORTED);
  if (cfg->kv_dtype != EAGLE3_KV_F32 && cfg->kv_dtype != EAGLE3_KV_BF16 && cfg->kv_dtype != EAGLE3_KV_Q8Q5)
    return bad("unknown kv_dtype", EAGLE3_E_INVAL);
  if (cfg->kv_dtype == EAGLE3_KV_Q8Q5 && cfg->max_seqs != 1)
    return bad("quantized KV: batch-1 drafting only (max_seqs 1)", EAGLE3_E_UNSUPPORTED);
  if (cfg->weight_format != EAGLE3_WEIGHTS_BF16 && cfg->weight_format != EAGLE3_WEIGHTS_I4)
    return bad("unknown weight_format", EAGLE3_E_INVAL);
  if (cfg->append_act != EAGLE3_APPEND_DEFAULT && cfg->append_act != EAGLE3_APPEND_BF16 &&
      cfg->append_act != EAGLE3_APPEND_SPLIT && cfg->append_act != EAGLE3_APPEND_F16)
    return bad("unknown append_act", EAGLE3_E_INVAL);
  if (cfg->token_table != EAGLE3_TABLE_DEFAULT && cfg->token_table != EAGLE3_TABLE_OFF &&
      cfg->token_table != EAGLE3_TABLE_ON)
    return bad("unknown token_table", EAGLE3_E_INVAL);
  if (cfg->append_act == EAGLE3_APPEND_F16 && cfg->weight_format != EAGLE3_WEIGHTS_BF16)
    return bad("fp16 teacher-forced activations need bf16 weights", EAGLE3_E_UNSUPPORTED);
  if (cfg->weight_format == EAGLE3_WEIGHTS_I4) {
    if (cfg->max_seqs != 1) return bad("int4 weights: batch-1 drafting only (max_seqs 1)", EAGLE3_E_UNSUPPORTED);
    if (cfg->n_embd % 32 || (int64_t(cfg->n_head) * cfg->head_dim) % 32 || cfg->n_ff % 32)
      return bad("int4 weights need input widths that are multiples of 32", EAGLE3_E_UNSUPPORTED);
    // the int4 GEMVs stage fp32 x and its fixed-point planes: 6.125 bytes per input
    const int64_t n = cfg->n_embd, kmax = std::max<int64_t>(
        {3 * n, int64_t(cfg->n_head) * cfg->head_dim, int64_t(cfg->n_ff)});
    if (kmax * 49 / 8 > kMaxLdsBytes || n * 98 / 8 > kMaxLdsBytes)
      return bad("int4 weights: an activation vector exceeds the LDS staging limit", EAGLE3_E_UNSUPPORTED);
  }
  {  // the GEMV kernels stage a whole fp32 activation vector in LDS
    const int64_t n = cfg->n_embd, kmax = std::max<int64_t>(
        {3 * n, 2 * n, int64_t(cfg->n_head) * cfg->head_dim, int64_t(cfg->n_ff)});
    if (kmax * 4 > kMaxStageBytes) return bad("an activation vector exceeds the LDS staging limit", EAGLE3_E_UNSUPPORTED);
  }
  return EAGLE3_OK;
}

// rotary-pair order of one head: position p -> source dim
int rope_src_dim(int p, int rot) {
  if (p >= rot) return p;
  return (p & 1) ? (p >> 1) + rot / 2 : (p >> 1);
}

}  // namespace

extern "C" {

int eagle3_resolve_rope_dim(int32_t rotary_dim, float partial_factor, int32_t head_dim,
                            int32_t* out) {
  if (!out) return EAGLE3_E_INVAL;
  if (head_dim <= 0 || (head_dim & 1)) return EAGLE3_E_INVAL;
  if (rotary_dim >= 0) {
    if (rotary_dim == 0 || rotary_dim > head_dim || (rotary_dim & 1)) return EAGLE3_E_UNSUPPORTED;
    *out = rotary_dim;
    return EAGLE3_OK;
  }
  if (partial_factor >= 0.f || std::isnan(partial_factor)) {
    const double f = partial_factor;
    if (!(std::isfinite(f) && f > 0.0 && f <= 1.0)) {  // malformed: full width
      *out = head_dim;
      return EAGLE3_OK;
    }
    const double dims = f * double(head_dim);
    const double r = std::nearbyint(dims);
    if (std::fabs(dims - r) > 1e-4 || r <= 0.0 || (int64_t(r) & 1)) return EAGLE3_E_UNSUPPORTED;
    *out = int32_t(r);
    return EAGLE3_OK;
  }
  *out = head_dim;
  return EAGLE3_OK;
}

int eagle3_load(const eagle3_config* cfg, const eagle3_weights* w, void* stream,
                eagle3_ctx** out) {
  g_load_error.clear();
  if (!out) return set_err(nullptr, EAGLE3_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!cfg || !w) return set_err(nullptr, EAGLE3_E_INVAL, "config or weights is NULL");
  const char* why = nullptr;
  int rc = validate_config(cfg, &why);
  if (rc) return set_err(nullptr, rc, why);
  const void* ptrs[14] = {w->fc, w->input_layernorm, w->hidden_norm, w->q_proj, w->k_proj,
                          w->v_proj, w->o_proj, w->post_attention_layernorm, w->gate_proj,
                          w->up_proj, w->down_proj, w->norm, w->lm_head, w->embed};
  static const char* names[14] = {"fc", "input_layernorm", "hidden_norm", "q_proj", "k_proj",
                                  "v_proj", "o_proj", "post_attention_layernorm", "gate_proj",
                                  "up_proj", "down_proj", "norm", "lm_head", "embed"};
  for (int i = 0; i < 14; ++i)
    if (!ptrs[i]) return set_err(nullptr, EAGLE3_E_INVAL, std::string(names[i]) + " is NULL");
  if (!w->d2t_host) return set_err(nullptr, EAGLE3_E_INVAL, "d2t is NULL");

  const int64_t n = cfg->n_embd, nh = cfg->n_head, nkv = cfg->n_head_kv, hd = cfg->head_dim;
  const int64_t qd = nh * hd, kvd = nkv * hd, ff = cfg->n_ff, dv = cfg->draft_vocab,
                vt = cfg->target_vocab;
  const int64_t want[14][2] = {{n, 3 * n}, {n, 1},  {n, 1},  {qd, 2 * n}, {kvd, 2 * n},
                               {kvd, 2 * n}, {n, qd}, {n, 1},  {ff, n},     {ff, n},
                               {n, ff},     {n, 1},  {dv, n}, {vt, n}};
  for (int i = 0; i < 14; ++i)
    if (w->shape[i][0] != want[i][0] || w->shape[i][1] != want[i][1]) {
      char buf[160];
      snprintf(buf, sizeof buf, "%s: declared [%lld, %lld], geometry implies [%lld, %lld]",
               names[i], (long long)w->shape[i][0], (long long)w->shape[i][1],
               (long long)want[i][0], (long long)want[i][1]);
      return set_err(nullptr, EAGLE3_E_SHAPE, buf);
    }
  if (w->d2t_len != dv) return set_err(nullptr, EAGLE3_E_SHAPE, "d2t length != draft_vocab");
  std::vector<int32_t> d2t_i32((size_t)dv);
  for (int64_t i = 0; i < dv; ++i) {
    const int64_t t = i + w->d2t_host[i];
    if (t < 0 || t >= vt) return set_err(nullptr, EAGLE3_E_INVAL, "d2t maps outside the target vocabulary");
    d2t_i32[size_t(i)] = int32_t(w->d2t_host[i]);
  }

  eagle3_ctx* c = new (std::nothrow) eagle3_ctx();
  if (!c) return set_err(nullptr, EAGLE3_E_OOM, "host allocation failed");
  c->cfg = *cfg;
  c->n = int(n); c->nh = int(nh); c->nkv = int(nkv); c->hd = int(hd);
  c->qd = int(qd); c->kvd = int(kvd); c->ff = int(ff); c->dv = int(dv); c->vt = int(vt);
  c->rot = cfg->rope_dim;
  c->cap = cfg->max_ctx + 1;
  // quantized regions hold a multiple of 16 rows: their decode attention reads whole
  // 16-row tiles (rows past T stay finite: the regions are zeroed below)
  if (cfg->kv_dtype == EAGLE3_KV_Q8Q5) c->cap = (c->cap + 15) / 16 * 16;
  c->ledger = e3::Ledger(cfg->max_ctx, cfg->max_seqs, cfg->max_gamma);
  hipStream_t s = as_stream(stream);

  auto fail = [&](int code) {
    g_load_error = c->err;
    (void)hipDeviceSynchronize();
    free_all(c);
    delete c;
    return code;
  };
#define E3_TRY(x)            \
  do {                       \
    int _rc = (x);           \
    if (_rc) return fail(_rc); \
  } while (0)
#define E3_TRYH(x, what)                                  \
  do {                                                    \
    hipError_t _e = (x);                                  \
    if (_e != hipSuccess) return fail(hip_fail(c, _e, what)); \
  } while (0)

  E3_TRYH(hipGetDevice(&c->device), "hipGetDevice");
  const size_t N_qkv = size_t(qd + 2 * kvd);
  E3_TRY(dalloc(c, &c->w_fc, size_t(n) * 3 * n));
  E3_TRY(dalloc(c, &c->w_qkv, N_qkv * 2 * n));
  E3_TRY(dalloc(c, &c->w_o, size_t(n) * qd));
  E3_TRY(dalloc(c, &c->w_gu, size_t(2 * ff) * n));
  E3_TRY(dalloc(c, &c->w_d, size_t(n) * ff));
  E3_TRY(dalloc(c, &c->w_lm, size_t(dv) * n));
  E3_TRY(dalloc(c, &c->embed, size_t(vt) * n));
  E3_TRY(dalloc(c, &c->nrm_in, size_t(n)));
  E3_TRY(dalloc(c, &c->nrm_hid, size_t(n)));
  E3_TRY(dalloc(c, &c->nrm_post, size_t(n)));
  E3_TRY(dalloc(c, &c->nrm_fin, size_t(n)));
  E3_TRY(dalloc(c, &c->d2t, size_t(dv)));
  E3_TRY(dalloc(c, &c->status, 1));
  c->kv_f32 = cfg->kv_dtype == EAGLE3_KV_F32;
  c->kv_q = cfg->kv_dtype == EAGLE3_KV_Q8Q5;
  c->kv_esize = c->kv_f32 ? 4 : (c->kv_q ? 1 : 2);
  c->kv_seq_elems = c->kv_q ? 2 * e3::kvq_region_bytes(int(c->nkv), c->cap, int(c->hd))
                            : size_t(2) * kvd * size_t(c->cap);
  if (c->kv_q) E3_TRY(dalloc(c, &c->kv_stage, size_t(2) * kvd));
  E3_TRY(dalloc(c, &c->kv, c->kv_seq_elems * size_t(cfg->max_seqs) * c->kv_esize));
  if (c->kv_q)
    E3_TRYH(hipMemsetAsync(c->kv, 0, c->kv_seq_elems * size_t(cfg->max_seqs) * c->kv_esize, s), "kv zero");

  E3_TRY(dalloc(c, &c->x1, size_t(n)));
  E3_TRY(dalloc(c, &c->x1w, size_t(n)));
  E3_TRY(dalloc(c, &c->act, size_t(ff)));
  E3_TRY(dalloc(c, &c->q, size_t(qd)));
  E3_TRY(dalloc(c, &c->ao, size_t(qd)));
  const size_t smax = size_t(e3::attn_max_splits(c->cap, c->hd, c->nkv));
  E3_TRY(dalloc(c, &c->part_o, size_t(nh) * smax * hd));
  E3_TRY(dalloc(c, &c->part_ml, size_t(nh) * smax * 2));
  const bool wi4 = cfg->weight_format == EAGLE3_WEIGHTS_I4;
  c->gcfg[e3::kGemvEncode] = e3::gemv_pick(e3::kGemvEncode, int(n), int(3 * n), wi4);
  c->gcfg[e3::kGemvQkv] = e3::gemv_pick(e3::kGemvQkv, int(qd + 2 * kvd), int(n), wi4);
  c->gcfg[e3::kGemvO] = e3::gemv_pick(e3::kGemvO, int(n), int(qd), wi4);
  c->gcfg[e3::kGemvGateUp] = e3::gemv_pick(e3::kGemvGateUp, int(2 * ff), int(n), wi4);
  c->gcfg[e3::kGemvDown] = e3::gemv_pick(e3::kGemvDown, int(n), int(ff), wi4);
  c->gcfg[e3::kGemvLmHead] = e3::gemv_pick(e3::kGemvLmHead, int(dv), int(n), wi4);
  E3_TRY(gemv_config_override(c));
  c->lm_grid = e3::lmhead_grid(int(dv), c->gcfg[e3::kGemvLmHead]);
  for (int i = 0; i < 3; ++i) {
    eagle3_ctx::GBuf& b = c->gb[i];
    b.count = e3::gemv_grid(int(n), c->gcfg[i == 0 ? e3::kGemvEncode : e3::kGemvDown]);
    E3_TRY(dalloc(c, &b.y, size_t(n)));
    E3_TRY(dalloc(c, &b.w_hid, size_t(n)));
    E3_TRY(dalloc(c, &b.w_norm, size_t(n)));
    E3_TRY(dalloc(c, &b.ssq, size_t(b.count)));
  }
  c->x1_count = e3::gemv_grid(int(n), c->gcfg[e3::kGemvO]);
  E3_TRY(dalloc(c, &c->x1_ssq, size_t(c->x1_count)));
  E3_TRY(dalloc(c, &c->lm_pv, size_t(c->lm_grid)));
  E3_TRY(dalloc(c, &c->lm_pi, size_t(c->lm_grid)));
  E3_TRY(dalloc(c, &c->lm_pt, size_t(c->lm_grid)));
  E3_TRY(dalloc(c, &c->tok_slots, size_t(cfg->max_gamma) + 1));
  E3_TRY(dalloc(c, &c->bnd_y, size_t(cfg->max_seqs) * n));
  E3_TRY(dalloc(c, &c->bnd_w, size_t(cfg->max_seqs) * n));
  E3_TRY(dalloc(c, &c->bnd_ssq, size_t(cfg->max_seqs)));
  c->cap_local = c->kv_q ? (cfg->max_gamma + 15) / 16 * 16 : cfg->max_gamma;
  c->kv_local_elems = c->kv_q ? 2 * e3::kvq_region_bytes(int(c->nkv), c->cap_local, int(c->hd))
                             : size_t(2) * c->nkv * c->cap_local * c->hd;
  E3_TRY(dalloc(c, &c->kv_local, size_t(cfg->max_seqs) * c->kv_local_elems * c->kv_esize));
  if (c->kv_q)
    E3_TRYH(hipMemsetAsync(c->kv_local, 0, size_t(cfg->max_seqs) * c->kv_local_elems * c->kv_esize, s),
            "local kv zero");
  E3_TRY(dalloc(c, &c->inv_freq, size_t(c->rot / 2)));

  // 4096-row passes: at the 5120-wide drafter W_fc's 256 x 320 output tiles then
  // number 256, one per CU, with no K split
  c->tf_rows = c->cap < 4096 ? c->cap : 4096;
  {  // small appends use split-K GEMV partials [splits][16][N]; large ones [splits][T][N]
    const size_t f_small = size_t(16) * n * size_t((3 * n + 511) / 512);
    const size_t p_small = size_t(16) * 2 * kvd * size_t((2 * n + 511) / 512);
    // MFMA appends: up to 4 K-split partials of a long pass, 16 of a short one
    // (<= 256 rows)
    const size_t big = std::max(size_t(c->tf_rows) * 4, size_t(256) * 16);
    c->tf_F_cap = std::max(big * n, f_small);
    c->tf_P_cap = std::max(big * 2 * kvd, p_small);
  }
  E3_TRY(dalloc(c, &c->tf_A, size_t(c->tf_rows) * 3 * n));
  E3_TRY(dalloc(c, &c->tf_cat16, size_t(c->tf_rows) * 2 * n));
  // the default: one fp16 product with bf16 weights, split bf16 terms with int4 weights
  const int32_t act = cfg->append_act != EAGLE3_APPEND_DEFAULT ? cfg->append_act
                      : cfg->weight_format == EAGLE3_WEIGHTS_BF16 ? EAGLE3_APPEND_F16
                                                                   : EAGLE3_APPEND_SPLIT;
  c->tf_f16 = act == EAGLE3_APPEND_F16;
  c->tf_split = act == EAGLE3_APPEND_SPLIT;
  if (c->tf_f16) {
    E3_TRY(dalloc(c, &c->w_fc16, size_t(n) * 3 * n));
    E3_TRY(dalloc(c, &c->w_kv16, size_t(2 * kvd) * 2 * n));
  }
  if (c->tf_split) {  // fp32-grade K/V rows
    E3_TRY(dalloc(c, &c->tf_A_lo, size_t(c->tf_rows) * 3 * n));
    E3_TRY(dalloc(c, &c->tf_cat16_lo, size_t(c->tf_rows) * 2 * n));
  }
  E3_TRY(dalloc(c, &c->tf_cat32, size_t(16) * 2 * n));
  E3_TRY(dalloc(c, &c->tf_F, c->tf_F_cap));
  E3_TRY(dalloc(c, &c->tf_P, c->tf_P_cap));

  if (cfg->max_seqs > 1) {
    using e3::kBatchRows;
    c->bp_enc = e3::bgemm_plan(int(n), int(3 * n), e3::kBEpiPartial);
    c->bp_qkv = e3::bgemm_plan(int(N_qkv), int(2 * n), e3::kBEpiPartial);
    c->bp_o = e3::bgemm_plan(int(n), int(qd), e3::kBEpiPartial);
    c->bp_gu = e3::bgemm_plan(int(2 * ff), int(n), e3::kBEpiSilu);
    c->bp_d = e3::bgemm_plan(int(n), int(ff), e3::kBEpiPartial);
    c->bp_lm = e3::bgemm_plan(int(dv), int(n), e3::kBEpiArgmax);
    auto tplan = [&](int64_t N, int64_t K) {
      e3::GemmPlan p{0, 0};
      if (K % 64 == 0) p = e3::gemm_plan(kBatchRows, int(N), int(K));
      return p;
    };
    c->tp_enc = tplan(n, 3 * n);
    c->tp_qkv = tplan(N_qkv, 2 * n);
    c->tp_o = tplan(n, qd);
    c->tp_gu = tplan(2 * ff, n);
    c->tp_d = tplan(n, ff);
    c->tp_lm = tplan(dv, n);
    // (helpers return the code; E3_TRY, which frees the context, runs at the call)
    auto tiled = [&](uint16_t** t, const e3::GemmPlan& p, int64_t N, int64_t K) -> int {
      return p.splits ? dalloc(c, t, e3::tiled_weight_elems(int(N), int(K))) : EAGLE3_OK;
    };
    E3_TRY(tiled(&c->bt_enc, c->tp_enc, n, 3 * n));
    E3_TRY(tiled(&c->bt_qkv, c->tp_qkv, N_qkv, 2 * n));
    E3_TRY(tiled(&c->bt_o, c->tp_o, n, qd));
    E3_TRY(tiled(&c->bt_gu, c->tp_gu, 2 * ff, n));
    E3_TRY(tiled(&c->bt_d, c->tp_d, n, ff));
    E3_TRY(tiled(&c->bt_lm, c->tp_lm, dv, n));
    // lm_head candidates per row: one per 128 weight rows from the fused epilogue of an
    // unsplit skinny GEMM, one per 2048 columns from the partials otherwise
    c->b_ncand = c->tp_lm.splits == 1 ? e3::sgemm_tiles(int(dv))
                 : c->tp_lm.splits ? e3::bcand_count(int(dv)) : c->bp_lm.blocks;
    c->bld_a = int(3 * n);
    c->bld_b = int(std::max(qd, ff));
    size_t pmax = 0;
    auto planes = [](const e3::GemmPlan& tp, const e3::BGemmPlan& bp, bool fused) {
      return size_t(tp.splits ? tp.splits : (fused ? 0 : bp.splits));
    };
    pmax = std::max(pmax, planes(c->tp_enc, c->bp_enc, false) * kBatchRows * size_t(n));
    pmax = std::max(pmax, planes(c->tp_qkv, c->bp_qkv, false) * kBatchRows * size_t(N_qkv));
    pmax = std::max(pmax, planes(c->tp_o, c->bp_o, false) * kBatchRows * size_t(n));
    pmax = std::max(pmax, planes(c->tp_d, c->bp_d, false) * kBatchRows * size_t(n));
    // gate/up and lm_head write partials only when split (one split: fused epilogues)
    auto fused_planes = [](const e3::GemmPlan& tp) { return size_t(tp.splits > 1 ? tp.splits : 0); };
    pmax = std::max(pmax, fused_planes(c->tp_gu) * kBatchRows * size_t(2 * ff));
    pmax = std::max(pmax, fused_planes(c->tp_lm) * kBatchRows * size_t(dv));
    const size_t bsp = size_t(e3::attn_batch_max_splits(c->cap, c->hd, c->kv_f32));
    E3_TRY(dalloc(c, &c->bx_a_hi, size_t(kBatchRows) * c->bld_a));
    E3_TRY(dalloc(c, &c->bx_a_lo, size_t(kBatchRows) * c->bld_a));
    E3_TRY(dalloc(c, &c->bx_b_hi, size_t(kBatchRows) * c->bld_b));
    E3_TRY(dalloc(c, &c->bx_b_lo, size_t(kBatchRows) * c->bld_b));
    E3_TRY(dalloc(c, &c->b_P, pmax));
    E3_TRY(dalloc(c, &c->b_G, size_t(kBatchRows) * n));
    E3_TRY(dalloc(c, &c->b_X1, size_t(kBatchRows) * n));
    E3_TRY(dalloc(c, &c->b_q, size_t(kBatchRows) * qd));
    E3_TRY(dalloc(c, &c->b_po, size_t(kBatchRows) * nh * bsp * hd));
    E3_TRY(dalloc(c, &c->b_pml, size_t(kBatchRows) * nh * bsp * 2));
    E3_TRY(dalloc(c, &c->b_cand_v, size_t(kBatchRows) * c->b_ncand));
    E3_TRY(dalloc(c, &c->b_cand_i, size_t(kBatchRows) * c->b_ncand));
    E3_TRY(dalloc(c, &c->b_logits, size_t(kBatchRows) * dv));
    E3_TRY(dalloc(c, &c->bx_z_hi, size_t(kBatchRows) * n));
    E3_TRY(dalloc(c, &c->bx_z_lo, size_t(kBatchRows) * n));
    E3_TRY(dalloc(c, &c->bx_h_hi, size_t(kBatchRows) * n));
    E3_TRY(dalloc(c, &c->bx_h_lo, size_t(kBatchRows) * n));
  }

  // zero state
  E3_TRYH(hipMemsetAsync(c->status, 0, 4, s), "clear status");
  E3_TRYH(hipMemsetAsync(c->kv, 0, c->kv_seq_elems * size_t(cfg->max_seqs) * c->kv_esize, s),
          "memset kv");

  // weights: straight copies
  auto cp = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  };
  E3_TRYH(cp(c->w_fc, w->fc, size_t(n) * 3 * n * 2), "copy fc");
  E3_TRYH(cp(c->w_o, w->o_proj, size_t(n) * qd * 2), "copy o_proj");
  E3_TRYH(cp(c->w_d, w->down_proj, size_t(n) * ff * 2), "copy down_proj");
  E3_TRYH(cp(c->w_lm, w->lm_head, size_t(dv) * n * 2), "copy lm_head");
  E3_TRYH(cp(c->embed, w->embed, size_t(vt) * n * 2), "copy embed");
  E3_TRYH(e3::launch_bf16_to_f32((const uint16_t*)w->input_layernorm, c->nrm_in, int(n), s), "norm");
  E3_TRYH(e3::launch_bf16_to_f32((const uint16_t*)w->hidden_norm, c->nrm_hid, int(n), s), "norm");
  E3_TRYH(e3::launch_bf16_to_f32((const uint16_t*)w->post_attention_layernorm, c->nrm_post, int(n), s), "norm");
  E3_TRYH(e3::launch_bf16_to_f32((const uint16_t*)w->norm, c->nrm_fin, int(n), s), "norm");
  E3_TRYH(hipMemcpyAsync(c->d2t, d2t_i32.data(), size_t(dv) * 4, hipMemcpyHostToDevice, s), "copy d2t");
  std::vector<double> invf((size_t)(c->rot / 2));
  for (int i = 0; i < c->rot / 2; ++i)
    invf[size_t(i)] = std::pow(double(cfg->rope_theta), -2.0 * double(i) / double(c->rot));
  E3_TRYH(hipMemcpyAsync(c->inv_freq, invf.data(), invf.size() * sizeof(double), hipMemcpyHostToDevice, s),
          "copy inv_freq");

  // repacks by row gathers: qkv (rotary pairs adjacent), gate/up interleaved
  {
    std::vector<int32_t> dst, src;
    const size_t maxrows = std::max<size_t>(size_t(qd), size_t(ff));
    int32_t* maps = nullptr;
    E3_TRY(dalloc(c, &maps, 2 * maxrows));
    auto gather = [&](uint16_t* D, const void* S, int row_len) -> int {
      hipError_t e = hipMemcpyAsync(maps, dst.data(), dst.size() * 4, hipMemcpyHostToDevice, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(maps + maxrows, src.data(), src.size() * 4, hipMemcpyHostToDevice, s);
      if (e == hipSuccess)
        e = e3::launch_gather_rows(D, (const uint16_t*)S, maps, maps + maxrows, int(dst.size()),
                                   row_len, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);  // host maps are reused
      return e == hipSuccess ? EAGLE3_OK : hip_fail(c, e, "repack");
    };
    auto head_perm = [&](int64_t heads, int64_t row_off) {
      dst.clear(); src.clear();
      for (int64_t h = 0; h < heads; ++h)
        for (int p = 0; p < hd; ++p) {
          dst.push_back(int32_t(row_off + h * hd + p));
          src.push_back(int32_t(h * hd + rope_src_dim(p, c->rot)));
        }
    };
    head_perm(nh, 0);
    E3_TRY(gather(c->w_qkv, w->q_proj, int(2 * n)));
    head_perm(nkv, qd);
    E3_TRY(gather(c->w_qkv, w->k_proj, int(2 * n)));
    E3_TRYH(cp(c->w_qkv + size_t(qd + kvd) * 2 * n, w->v_proj, size_t(kvd) * 2 * n * 2), "copy v");
    dst.clear(); src.clear();
    for (int64_t i = 0; i < ff; ++i) { dst.push_back(int32_t(2 * i)); src.push_back(int32_t(i)); }
    E3_TRY(gather(c->w_gu, w->gate_proj, int(n)));
    for (int64_t i = 0; i < ff; ++i) dst[size_t(i)] = int32_t(2 * i + 1);
    E3_TRY(gather(c->w_gu, w->up_proj, int(n)));
  }
  if (c->tf_f16) {  // fp16 copies (x 2^8, exact) of the weights the MFMA appends multiply
    E3_TRYH(e3::launch_bf16_to_f16_x256(c->w_fc, c->w_fc16, size_t(n) * 3 * n, c->status, s), "fp16 fc");
    E3_TRYH(e3::launch_bf16_to_f16_x256(c->w_qkv + size_t(qd) * 2 * n, c->w_kv16, size_t(2 * kvd) * 2 * n,
                                        c->status, s),
            "fp16 kv");
  }
  {  // the batched projections' step-tiled weights (after the repacks)
    auto tile = [&](uint16_t* t, const uint16_t* w, int64_t N, int64_t K) -> int {
      const hipError_t e = t ? e3::launch_tile_weights(w, int(N), int(K), t, s) : hipSuccess;
      return e == hipSuccess ? EAGLE3_OK : hip_fail(c, e, "tile weights");
    };
    E3_TRY(tile(c->bt_enc, c->w_fc, n, 3 * n));
    E3_TRY(tile(c->bt_qkv, c->w_qkv, N_qkv, 2 * n));
    E3_TRY(tile(c->bt_o, c->w_o, n, qd));
    E3_TRY(tile(c->bt_gu, c->w_gu, 2 * ff, n));
    E3_TRY(tile(c->bt_d, c->w_d, n, ff));
    E3_TRY(tile(c->bt_lm, c->w_lm, dv, n));
  }
  if (cfg->weight_format == EAGLE3_WEIGHTS_I4) {
    c->i4 = true;
    // (returns the code; E3_TRY, which frees the context, runs at the call)
    auto quant = [&](const uint16_t* W, int64_t rows, int64_t K, eagle3_ctx::I4W* m) -> int {
      if (int rc = dalloc(c, &m->q, size_t(rows) * size_t(K) / 2)) return rc;
      if (int rc = dalloc(c, &m->s, size_t(rows) * size_t(K) / 32)) return rc;
      const hipError_t e = e3::launch_quant_i4(W, int(rows), int(K), m->q, m->s, s);
      return e == hipSuccess ? EAGLE3_OK : hip_fail(c, e, "int4 quantize");
    };
    E3_TRY(quant(c->w_fc, n, 3 * n, &c->i4_fc));
    E3_TRY(quant(c->w_qkv, N_qkv, 2 * n, &c->i4_qkv));
    E3_TRY(quant(c->w_o, n, qd, &c->i4_o));
    E3_TRY(quant(c->w_gu, 2 * ff, n, &c->i4_gu));
    E3_TRY(quant(c->w_d, n, ff, &c->i4_d));
    E3_TRY(quant(c->w_lm, dv, n, &c->i4_lm));
    E3_TRY(dalloc(c, &c->i4_fc_lo, size_t(n) * 3 * n));
    // every QKV row as the int4 weights' (hi, lo) halves: hi over the bf16 rows (Q
    // rows included: in this form only the token table reads them), lo beside them
    E3_TRY(dalloc(c, &c->i4_qkv_lo, N_qkv * 2 * n));
    c->i4_kv_lo = c->i4_qkv_lo + size_t(qd) * 2 * n;
    E3_TRYH(e3::launch_dequant_i4_split(c->i4_fc.q, c->i4_fc.s, int(n), int(3 * n), c->w_fc, c->i4_fc_lo, s),
            "int4 fc split");
    E3_TRYH(e3::launch_dequant_i4_split(c->i4_qkv.q, c->i4_qkv.s, int(N_qkv), int(2 * n), c->w_qkv, c->i4_qkv_lo,
                                        s),
            "int4 qkv split");
  }
  if (cfg->token_table != EAGLE3_TABLE_OFF) {
    // the token table: passes of T tokens, input_layernorm * E / rms(E) as (hi, lo) bf16
    // planes in tf_A, one MFMA GEMM against the embedding half of the repacked W_qkv
    // (int4: a second against the weights' lo halves, summed through tf_F)
    E3_TRY(dalloc(c, &c->tok_tab, size_t(vt) * N_qkv));
    E3_TRY(dalloc(c, &c->tok_ss, size_t(vt)));
    if (!c->i4) {
      // the hidden half as its own matrix: read in place, 8 KB-aligned halves of 16 KB
      // rows, it streamed at about 60 % of the contiguous rate (measured in the fused
      // lm_head launch: 55.6 against 51.5 us at the Qwen3-8B shape)
      E3_TRY(dalloc(c, &c->w_qkv_h, N_qkv * n));
      E3_TRYH(hipMemcpy2DAsync(c->w_qkv_h, size_t(n) * 2, c->w_qkv + n, size_t(2 * n) * 2, size_t(n) * 2, N_qkv,
                               hipMemcpyDeviceToDevice, s),
              "hidden-half copy");
    }
    if (!c->kv_q) {
      // EAGLE3_DEFER_QKV=0 keeps the fused QKV kernel (for comparison)
      const char* dq = std::getenv("EAGLE3_DEFER_QKV");
      c->defer_qkv = !(dq && dq[0] == '0') && c->lm_grid <= e3::kDqMaxCandidates;
      if (c->defer_qkv) E3_TRY(dalloc(c, &c->hsum, N_qkv));
      const char* bq = std::getenv("EAGLE3_BOUNDARY_QH");
      if (c->defer_qkv && !(bq && bq[0] == '0')) {
        E3_TRY(dalloc(c, &c->bnd_hsum, size_t(cfg->max_seqs) * N_qkv));
        c->bnd_hsum_ok.assign(size_t(cfg->max_seqs), 0);
      }
    }
    E3_TRYH(e3::launch_tok_ss(c->embed, int(vt), int(n), c->tok_ss, s), "token table norms");
    int T = c->tf_rows;
    if (c->i4) T = int(std::min<size_t>(size_t(T), c->tf_F_cap / N_qkv));
    if (T < 1) return fail(set_err(c, EAGLE3_E_UNSUPPORTED, "token table: no room for a pass"));
    uint16_t* A_hi = c->tf_A;
    uint16_t* A_lo = c->tf_A + size_t(T) * n;  // tf_A holds 3 n values per row
    for (int64_t r0 = 0; r0 < vt; r0 += T) {
      const int rows = int(std::min<int64_t>(T, vt - r0));
      E3_TRYH(e3::launch_pack_embed(c->embed, c->nrm_in, c->tok_ss, c->cfg.rms_eps, int(r0), rows, int(n), A_hi, A_lo, s),
              "token table pack");
      e3::GemmPlan p = e3::gemm_plan(rows, int(N_qkv), int(n));
      p.splits = 1;  // one plane: the table rows are written in place
      float* dst = c->tok_tab + size_t(r0) * N_qkv;
      E3_TRYH(e3::launch_gemm_bf16(A_hi, A_lo, int(n), c->w_qkv, int(2 * n), dst, rows, int(N_qkv), int(n), p, s),
              "token table gemm");
      if (c->i4) {
        E3_TRYH(e3::launch_gemm_bf16(A_hi, A_lo, int(n), c->i4_qkv_lo, int(2 * n), c->tf_F, rows, int(N_qkv),
                                     int(n), p, s),
                "token table gemm lo");
        E3_TRYH(e3::launch_add_f32(dst, c->tf_F, size_t(rows) * N_qkv, s), "token table sum");
      }
    }
  }
  E3_TRYH(hipStreamSynchronize(s), "load sync");
#undef E3_TRY
#undef E3_TRYH
  *out = c;
  return EAGLE3_OK;
}

int eagle3_free(eagle3_ctx* ctx) {
  if (!ctx) return EAGLE3_OK;
  (void)hipDeviceSynchronize();
  free_all(ctx);
  delete ctx;
  return EAGLE3_OK;
}

const char* eagle3_last_error(const eagle3_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_load_error.c_str();
}

size_t eagle3_verify_attention_workspace(int32_t M, int32_t n_head, int32_t n_head_kv,
                                         int32_t head_dim, int32_t ctx_rows, int32_t kv_dtype) {
  if (M < 1 || ctx_rows < 0 || n_head_kv < 1 || n_head < n_head_kv) return 0;
  return e3::attn_verify_workspace(M, n_head, n_head_kv, head_dim, ctx_rows, kv_dtype == EAGLE3_KV_F32);
}

int eagle3_verify_attention(const float* q_dev, const void* k_dev, const void* v_dev, int32_t kv_dtype,
                            int32_t cap, int32_t ctx_rows, int32_t M, int32_t n_head, int32_t n_head_kv,
                            int32_t head_dim, float* out_dev, void* workspace_dev, size_t workspace_bytes,
                            void* stream) {
  if (!q_dev || !k_dev || !v_dev || !out_dev || M < 1 || ctx_rows < 0 || cap < 1 ||
      int64_t(ctx_rows) + M > cap || n_head < 1 || n_head_kv < 1)
    return EAGLE3_E_INVAL;
  if (n_head % n_head_kv) return EAGLE3_E_SHAPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return EAGLE3_E_UNSUPPORTED;
  if (kv_dtype != EAGLE3_KV_F32 && kv_dtype != EAGLE3_KV_BF16) return EAGLE3_E_UNSUPPORTED;
  const int f32 = kv_dtype == EAGLE3_KV_F32;
  const size_t need = e3::attn_verify_workspace(M, n_head, n_head_kv, head_dim, ctx_rows, f32);
  e3::VerifyArgs a{};
  a.q = q_dev; a.k = k_dev; a.v = v_dev; a.kv_f32 = f32;
  a.cap = cap; a.ctx = ctx_rows; a.M = M;
  a.n_head = n_head; a.n_head_kv = n_head_kv; a.head_dim = head_dim;
  float* ws = static_cast<float*>(workspace_dev);
  const size_t po = need / sizeof(float) / size_t(head_dim + 2) * size_t(head_dim);  // part_o floats
  a.part_o = ws;
  a.part_ml = ws ? ws + po : nullptr;
  a.out = out_dev;
  const hipError_t e = e3::launch_attn_verify(a, ws ? workspace_bytes : 0, as_stream(stream));
  if (e == hipErrorInvalidValue) return EAGLE3_E_INVAL;
  return e == hipSuccess ? EAGLE3_OK : EAGLE3_E_HIP;
}

static_assert(EAGLE3_VERIFY_SCRATCH_BYTES == e3::kVerifyScratchBytes, "scratch size in the header");

int eagle3_verify_attention_noalloc(const float* q_dev, const void* k_dev, const void* v_dev,
                                    int32_t kv_dtype, int32_t cap, int32_t ctx_rows, int32_t M,
                                    int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                                    float* out_dev, void* stream) {
  g_load_error.clear();
  if (!q_dev || !k_dev || !v_dev || !out_dev || M < 1 || ctx_rows < 0 || cap < 1 ||
      int64_t(ctx_rows) + M > cap || n_head < 1 || n_head_kv < 1)
    return set_err(nullptr, EAGLE3_E_INVAL, "verify attention: bad argument");
  if (n_head % n_head_kv) return set_err(nullptr, EAGLE3_E_SHAPE, "n_head % n_head_kv != 0");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return set_err(nullptr, EAGLE3_E_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (kv_dtype != EAGLE3_KV_F32 && kv_dtype != EAGLE3_KV_BF16)
    return set_err(nullptr, EAGLE3_E_UNSUPPORTED, "kv_dtype must be EAGLE3_KV_F32 or EAGLE3_KV_BF16");
  const int f32 = kv_dtype == EAGLE3_KV_F32;
  const size_t need = e3::attn_verify_workspace(M, n_head, n_head_kv, head_dim, ctx_rows, f32);
  if (need > e3::kVerifyScratchBytes) {
    char buf[160];
    snprintf(buf, sizeof buf, "verify attention: %zu bytes of split partials exceed the %zu-byte static scratch",
             need, e3::kVerifyScratchBytes);
    return set_err(nullptr, EAGLE3_E_CAPACITY, buf);
  }
  void* ws = nullptr;
  hipError_t e = e3::verify_scratch_ptr(&ws);
  if (e != hipSuccess) return hip_fail(nullptr, e, "verify attention scratch");
  e3::VerifyArgs a{};
  a.q = q_dev; a.k = k_dev; a.v = v_dev; a.kv_f32 = f32;
  a.cap = cap; a.ctx = ctx_rows; a.M = M;
  a.n_head = n_head; a.n_head_kv = n_head_kv; a.head_dim = head_dim;
  const size_t po = need / sizeof(float) / size_t(head_dim + 2) * size_t(head_dim);  // part_o floats
  a.part_o = static_cast<float*>(ws);
  a.part_ml = static_cast<float*>(ws) + po;
  a.out = out_dev;
  e = e3::launch_attn_verify(a, e3::kVerifyScratchBytes, as_stream(stream));
  if (e == hipErrorInvalidValue) return set_err(nullptr, EAGLE3_E_INVAL, "verify attention: bad argument");
  return e == hipSuccess ? EAGLE3_OK : hip_fail(nullptr, e, "verify attention launch");
}

int eagle3_status(eagle3_ctx* ctx, uint32_t* flags) {
  if (!ctx || !flags) return EAGLE3_E_INVAL;
  hipError_t e = hipDeviceSynchronize();
  uint32_t v = 0;
  if (e == hipSuccess) e = hipMemcpy(&v, ctx->status, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(ctx->status, 0, 4);
  if (e != hipSuccess) return hip_fail(ctx, e, "status");
  *flags = v;
  return EAGLE3_OK;
}

int eagle3_kv_len(const eagle3_ctx* ctx, int32_t seq, int32_t* committed, int32_t* spec) {
  if (!ctx || !committed || !spec) return EAGLE3_E_INVAL;
  if (!ctx->ledger.valid_seq(seq)) return EAGLE3_E_INVAL;
  *committed = ctx->ledger.seq(seq).committed;
  *spec = ctx->ledger.seq(seq).spec;
  return EAGLE3_OK;
}

int eagle3_rewind(eagle3_ctx* ctx, int32_t seq, int32_t new_len) {
  if (!ctx) return EAGLE3_E_INVAL;
  const char* why = nullptr;
  int rc = ctx->ledger.check_rewind(seq, new_len, &why);
  if (rc) return set_err(ctx, rc, why);
  ctx->ledger.do_rewind(seq, new_len);
  return EAGLE3_OK;
}

int eagle3_kv_read(const eagle3_ctx* cctx, int32_t seq, int32_t row0, int32_t nrows, void* k_dev,
                   void* v_dev, void* stream) {
  eagle3_ctx* ctx = const_cast<eagle3_ctx*>(cctx);
  if (!ctx || !k_dev || !v_dev) return EAGLE3_E_INVAL;
  if (!ctx->ledger.valid_seq(seq)) return set_err(ctx, EAGLE3_E_INVAL, "bad sequence id");
  if (row0 < 0 || nrows < 0 || int64_t(row0) + nrows > ctx->cap)
    return set_err(ctx, EAGLE3_E_INVAL, "rows outside the allocation");
  if (nrows == 0) return EAGLE3_OK;
  hipStream_t s = as_stream(stream);
  if (ctx->kv_q) {  // quantized regions: dequantized to fp32
    E3_HIP(ctx, e3::launch_kvq_read(ctx->k_of(seq), ctx->v_of(seq), int(ctx->nkv), ctx->cap, int(ctx->hd),
                                    row0, nrows, static_cast<float*>(k_dev), static_cast<float*>(v_dev), s),
           "kv_read");
    return EAGLE3_OK;
  }
  // cache is [nkv][cap][hd]; output is [nrows][nkv][hd], same element type
  const size_t rowb = size_t(ctx->hd) * ctx->kv_esize;
  for (int half = 0; half < 2; ++half) {
    const char* base = static_cast<const char*>(half ? ctx->v_of(seq) : ctx->k_of(seq));
    char* dst = static_cast<char*>(half ? v_dev : k_dev);
    for (int h = 0; h < ctx->nkv; ++h) {
      E3_HIP(ctx,
             hipMemcpy2DAsync(dst + size_t(h) * rowb, size_t(ctx->nkv) * rowb,
                              base + (size_t(h) * ctx->cap + row0) * rowb, rowb, rowb,
                              size_t(nrows), hipMemcpyDeviceToDevice, s),
             "kv_read");
    }
  }
  return EAGLE3_OK;
}

int eagle3_weights_i4_read(const eagle3_ctx* cctx, int32_t matrix, void* codes_dev,
                           void* scales_dev, void* stream) {
  eagle3_ctx* ctx = const_cast<eagle3_ctx*>(cctx);
  if (!ctx || !codes_dev || !scales_dev) return EAGLE3_E_INVAL;
  if (!ctx->i4) return set_err(ctx, EAGLE3_E_STATE, "the weights are not int4");
  const int64_t n = ctx->n;
  const eagle3_ctx::I4W* m = nullptr;
  int64_t rows = 0, K = 0;
  switch (matrix) {
    case EAGLE3_I4_FC: m = &ctx->i4_fc; rows = n; K = 3 * n; break;
    case EAGLE3_I4_QKV: m = &ctx->i4_qkv; rows = ctx->qd + 2 * ctx->kvd; K = 2 * n; break;
    case EAGLE3_I4_O: m = &ctx->i4_o; rows = n; K = ctx->qd; break;
    case EAGLE3_I4_GATE_UP: m = &ctx->i4_gu; rows = 2 * ctx->ff; K = n; break;
    case EAGLE3_I4_DOWN: m = &ctx->i4_d; rows = n; K = ctx->ff; break;
    case EAGLE3_I4_LM_HEAD: m = &ctx->i4_lm; rows = ctx->dv; K = n; break;
    default: return set_err(ctx, EAGLE3_E_INVAL, "unknown matrix");
  }
  hipStream_t s = as_stream(stream);
  E3_HIP(ctx, hipMemcpyAsync(codes_dev, m->q, size_t(rows * K / 2), hipMemcpyDeviceToDevice, s),
         "int4 read");
  E3_HIP(ctx, hipMemcpyAsync(scales_dev, m->s, size_t(rows * K / 32) * 2, hipMemcpyDeviceToDevice, s),
         "int4 read");
  return EAGLE3_OK;
}

// ---- teacher-forced append over packed rows ----------------------------------
namespace {

struct AppendSeg {
  int seq, row0, T, pos0;
};

// The next rounds' boundary taps that come with an append: count rows of
// three fp32 streams [count][n]; row j is the boundary of sequence slot slots[j].
struct BndIn {
  const float* y[3] = {nullptr, nullptr, nullptr};
  std::vector<int32_t> slots;
  int count() const { return int(slots.size()); }
};

// Teacher-forced rows (segments of `total` packed rows) and then the boundary rows,
// in passes of up to tf_rows rows (at most kBndRows of them boundary rows): W_fc is
// streamed once per pass for all of its rows; the K/V projection, rotation and
// store run for the teacher-forced rows, the boundary rows end in the per-slot
// boundary features.
int append_rows(eagle3_ctx* c, const std::vector<AppendSeg>& segs, int total, const int32_t* tok,
                const float* a0, const float* a1, const float* a2, const BndIn& bi, hipStream_t s) {
  const int n = c->n, kvd2 = 2 * c->kvd;
  const int all = total + bi.count();
  size_t seg_i = 0;
  const int pass_rows = c->tf_rows;
  const int wsp = c->i4 ? 2 : 1;  // int4: each MFMA product twice, weights hi and lo
  for (int c0 = 0; c0 < all;) {
    int P = std::min(pass_rows, all - c0);
    const int T = std::max(0, std::min(total, c0 + P) - c0);  // teacher-forced rows of the pass
    int Tb = P - T;
    if (Tb > e3::kBndRows) {
      Tb = e3::kBndRows;
      P = T + Tb;
    }
    const int b0 = std::max(c0, total) - total;  // first boundary row of the pass
    e3::TapRowsB yb = e3::no_tap_rows_b();
    e3::BndOut bo{};
    const float *x0 = a0 + size_t(c0) * n, *x1 = a1 + size_t(c0) * n, *x2 = a2 + size_t(c0) * n;
    if (Tb > 0) {
      for (int k = 0; k < 3; ++k) yb.y[k] = bi.y[k] + size_t(b0) * n;
      yb.rows_x = T;
      if (T == 0) {
        x0 = yb.y[0];
        x1 = yb.y[1];
        x2 = yb.y[2];
      }
      bo.y = c->bnd_y;
      bo.yw = c->bnd_w;
      bo.ssq = c->bnd_ssq;
      bo.count = Tb;
      for (int j = 0; j < Tb; ++j) bo.slot[j] = bi.slots[size_t(b0 + j)];
      // a new boundary feature: its hidden-half sums are stale until this pass's
      // K/V launch computes them (below, when it does)
      if (c->bnd_hsum)
        for (int j = 0; j < Tb; ++j) c->bnd_hsum_ok[size_t(bo.slot[j])] = 0;
    }
    int sp1 = 1, sp2 = 1;
    size_t f_split = 0, p_split = 0;
    float p_scale = 1.0f;  // applied to the summed products of this pass
    if (P <= 16) {
      // weight-streaming path: every weight chunk applied to all rows of the pass
      {
        ProfScope ps(c, 7, s);
        E3_HIP(c, e3::launch_gemv_multi(c->wq(c->w_fc, c->i4_fc), c->ws(c->i4_fc), n, 3 * n, x0, x1,
                                        x2, n, P, c->tf_F, &sp1, s, yb),
               "fc gemv");
      }
      f_split = size_t(e3::gemv_multi_width(P)) * n;
      E3_HIP(c, e3::launch_tf_cat(c->status, c->tf_F, sp1, f_split, T, n, c->embed, c->vt, tok + c0, c->nrm_in,
                                  c->nrm_hid, c->cfg.rms_eps, nullptr, nullptr, c->tf_cat32, s, &bo),
             "tf cat");
      // the boundary row's hidden-half QKV sums ride in the K/V launch (one boundary
      // row with teacher-forced rows in the pass)
      if (T > 0 && Tb == 1 && c->bnd_hsum) {
        const int slot = bo.slot[0];
        e3::QhArgs q = c->qh_args(eagle3_ctx::GBuf{c->bnd_y + size_t(slot) * n, c->bnd_w + size_t(slot) * n,
                                                   nullptr, c->bnd_ssq + slot, 1});
        q.hsum = c->bnd_hsum + size_t(slot) * q.N;
        ProfScope ps(c, 8, s);
        E3_HIP(c, e3::launch_gemv_multi_qh(c->wq(c->w_qkv, c->i4_qkv, size_t(c->qd), 2 * n),
                                           c->ws(c->i4_qkv, size_t(c->qd), 2 * n), kvd2, 2 * n, c->tf_cat32, T,
                                           c->tf_P, &sp2, q, s),
               "kv gemv + boundary qkv hidden half");
        c->bnd_hsum_ok[size_t(slot)] = 1;
      } else if (T > 0) {
        ProfScope ps(c, 8, s);
        // the K and V rows of the fused QKV matrix
        E3_HIP(c, e3::launch_gemv_multi(c->wq(c->w_qkv, c->i4_qkv, size_t(c->qd), 2 * n),
                                        c->ws(c->i4_qkv, size_t(c->qd), 2 * n), kvd2, 2 * n,
                                        c->tf_cat32, nullptr, nullptr, 0, T, c->tf_P, &sp2, s),
               "kv gemv");
      }
      p_split = size_t(e3::gemv_multi_width(T > 0 ? T : 1)) * kvd2;
    } else {
      // MFMA path
      E3_HIP(c, e3::launch_pack_aux(x0, x1, x2, P, n, c->tf_A, c->tf_A_lo, s, yb, c->tf_f16, c->status),
             "pack aux");
      if (c->tf_f16) p_scale = 1.0f / 256.0f;  // the fp16 weight copies carry 2^8
      e3::GemmPlan p1 = e3::gemm_plan(P, n, 3 * n);
      while (p1.splits > 1 && size_t(wsp) * p1.splits * P * n > c->tf_F_cap) p1.splits /= 2;
      sp1 = p1.splits * wsp;
      {
        ProfScope ps(c, 7, s);
        E3_HIP(c, e3::launch_gemm_bf16(c->tf_A, c->tf_A_lo, 3 * n, c->tf_f16 ? c->w_fc16 : c->w_fc, 3 * n,
                                       c->tf_F, P, n, 3 * n, p1, s, c->tf_f16 != 0), "fc gemm");
        if (c->i4)  // the weights' low halves into the next split slots
          E3_HIP(c, e3::launch_gemm_bf16(c->tf_A, c->tf_A_lo, 3 * n, c->i4_fc_lo, 3 * n,
                                         c->tf_F + size_t(p1.splits) * P * n, P, n, 3 * n, p1, s),
                 "fc gemm lo");
      }
      f_split = size_t(P) * n;
      E3_HIP(c, e3::launch_tf_cat(c->status, c->tf_F, sp1, f_split, T, n, c->embed, c->vt, tok + c0, c->nrm_in,
                                  c->nrm_hid, c->cfg.rms_eps, c->tf_cat16, c->tf_cat16_lo, nullptr, s,
                                  &bo, p_scale, c->tf_f16),
             "tf cat");
      if (T > 0) {
        e3::GemmPlan p2 = e3::gemm_plan(T, kvd2, 2 * n);
        while (p2.splits > 1 && size_t(wsp) * p2.splits * T * kvd2 > c->tf_P_cap) p2.splits /= 2;
        sp2 = p2.splits * wsp;
        ProfScope ps(c, 8, s);
        E3_HIP(c, e3::launch_gemm_bf16(c->tf_cat16, c->tf_cat16_lo, 2 * n,
                                       c->tf_f16 ? c->w_kv16 : c->w_qkv + size_t(c->qd) * 2 * n, 2 * n,
                                       c->tf_P, T, kvd2, 2 * n, p2, s, c->tf_f16 != 0), "kv gemm");
        if (c->i4)
          E3_HIP(c, e3::launch_gemm_bf16(c->tf_cat16, c->tf_cat16_lo, 2 * n, c->i4_kv_lo, 2 * n,
                                         c->tf_P + size_t(p2.splits) * T * kvd2, T, kvd2, 2 * n, p2, s),
                 "kv gemm lo");
      }
      p_split = size_t(T) * kvd2;
    }
    if (T > 0) {
      // store the rows of this pass into each segment's cache rows, up to
      // kStoreSegs segments per launch
      e3::StoreSegs ss{};
      auto flush = [&]() -> int {
        if (ss.n == 0) return EAGLE3_OK;
        E3_HIP(c, e3::launch_tf_store(c->tf_P, sp2, p_split, ss, c->nkv, c->hd, c->rot, c->inv_freq,
                                      c->kv, c->kv_seq_elems, c->cap, c->kv_f32, s, c->kv_q, p_scale),
               "tf store");
        ss = e3::StoreSegs{};
        return EAGLE3_OK;
      };
      for (; seg_i < segs.size(); ++seg_i) {
        const AppendSeg& g = segs[seg_i];
        const int lo = std::max(g.row0, c0), hi = std::min(g.row0 + g.T, c0 + T);
        if (hi > lo) {
          if (ss.n == e3::kStoreSegs)
            if (int rc = flush()) return rc;
          ss.row0[ss.n] = lo - c0;
          ss.pos0[ss.n] = g.pos0 + (lo - g.row0);
          ss.slot[ss.n] = g.seq;
          ss.row0[++ss.n] = hi - c0;
        }
        if (g.row0 + g.T > c0 + T) break;  // continues in the next pass
      }
      if (int rc = flush()) return rc;
    }
    c0 += P;
  }
  return EAGLE3_OK;
}

// next-boundary tap pointers: all three or none
int check_next_taps(eagle3_ctx* c, const float* b0, const float* b1, const float* b2, bool* given) {
  *given = b0 || b1 || b2;
  if (*given && !(b0 && b1 && b2))
    return set_err(c, EAGLE3_E_INVAL, "next-boundary taps: give all three streams or none");
  if (*given && (!aligned16(b0) || !aligned16(b1) || !aligned16(b2)))
    return set_err(c, EAGLE3_E_INVAL, "tap pointers must be 16-byte aligned");
  return EAGLE3_OK;
}

}  // namespace

int eagle3_prefill(eagle3_ctx* ctx, int32_t seq, int32_t T, const int32_t* tok_dev,
                   const float* aux0_dev, const float* aux1_dev, const float* aux2_dev,
                   const float* next_aux0_dev, const float* next_aux1_dev,
                   const float* next_aux2_dev, void* stream) {
  if (!ctx) return EAGLE3_E_INVAL;
  const char* why = nullptr;
  int rc = ctx->ledger.check_prefill(seq, T, &why);
  if (rc) return set_err(ctx, rc, why);
  bool next = false;
  rc = check_next_taps(ctx, next_aux0_dev, next_aux1_dev, next_aux2_dev, &next);
  if (rc) return rc;
  if (T == 0 && !next) return EAGLE3_OK;
  if (T > 0) {
    if (!tok_dev || !aux0_dev || !aux1_dev || !aux2_dev)
      return set_err(ctx, EAGLE3_E_INVAL, "null input pointer");
    if (!aligned16(aux0_dev) || !aligned16(aux1_dev) || !aligned16(aux2_dev))
      return set_err(ctx, EAGLE3_E_INVAL, "tap pointers must be 16-byte aligned");
  }
  const int32_t start = ctx->ledger.seq(seq).committed;
  std::vector<AppendSeg> segs;
  if (T > 0) segs.push_back({seq, 0, T, start});
  BndIn bi;
  if (next) {
    bi.y[0] = next_aux0_dev;
    bi.y[1] = next_aux1_dev;
    bi.y[2] = next_aux2_dev;
    bi.slots.push_back(seq);
  }
  rc = append_rows(ctx, segs, T, tok_dev, aux0_dev, aux1_dev, aux2_dev, bi, as_stream(stream));
  if (rc) return rc;
  ctx->ledger.do_prefill(seq, T, next);
  return EAGLE3_OK;
}

int eagle3_rebuild_after_verify(eagle3_ctx* ctx, int32_t n_seq, const int32_t* seq_ids_host,
                                const int32_t* n_accepted_host, const int32_t* tok_dev,
                                const float* aux0_dev, const float* aux1_dev,
                                const float* aux2_dev, const float* next_aux0_dev,
                                const float* next_aux1_dev, const float* next_aux2_dev,
                                void* stream) {
  if (!ctx) return EAGLE3_E_INVAL;
  if (n_seq < 0 || (n_seq > 0 && (!seq_ids_host || !n_accepted_host)))
    return set_err(ctx, EAGLE3_E_INVAL, "bad sequence list");
  if (n_seq == 0) return EAGLE3_OK;
  if (!tok_dev || !aux0_dev || !aux1_dev || !aux2_dev)
    return set_err(ctx, EAGLE3_E_INVAL, "null input pointer");
  if (!aligned16(aux0_dev) || !aligned16(aux1_dev) || !aligned16(aux2_dev))
    return set_err(ctx, EAGLE3_E_INVAL, "tap pointers must be 16-byte aligned");
  bool next = false;
  int rc = check_next_taps(ctx, next_aux0_dev, next_aux1_dev, next_aux2_dev, &next);
  if (rc) return rc;
  std::vector<AppendSeg> segs;
  BndIn bi;
  int total = 0;
  for (int b = 0; b < n_seq; ++b) {
    const char* why = nullptr;
    const int s = seq_ids_host[b];
    rc = ctx->ledger.check_rebuild(s, n_accepted_host[b], &why);
    if (rc) return set_err(ctx, rc, why);
    for (int j = 0; j < b; ++j)
      if (seq_ids_host[j] == s) return set_err(ctx, EAGLE3_E_INVAL, "duplicate sequence id");
    segs.push_back({s, total, n_accepted_host[b] + 1, ctx->ledger.seq(s).committed});
    total += n_accepted_host[b] + 1;
    if (next) bi.slots.push_back(s);
  }
  if (next) {
    bi.y[0] = next_aux0_dev;
    bi.y[1] = next_aux1_dev;
    bi.y[2] = next_aux2_dev;
  }
  rc = append_rows(ctx, segs, total, tok_dev, aux0_dev, aux1_dev, aux2_dev, bi, as_stream(stream));
  if (rc) return rc;
  for (int b = 0; b < n_seq; ++b) ctx->ledger.do_rebuild(seq_ids_host[b], n_accepted_host[b], next);
  return EAGLE3_OK;
}

}  // extern "C"

namespace {

// Batched rounds: passes of up to 32 sequences; inside a pass each GEMM streams its
// weights once for all rows still drafting.
int draft_chain_batched(eagle3_ctx* c, int32_t n_seq, const int32_t* seq_ids,
                        const int32_t* btok, const float* a0, const float* a1, const float* a2,
                        bool stored, bool local, int32_t gamma, int32_t* out,
                        const std::vector<int32_t>& geff, const eagle3_debug* dbg, hipStream_t s) {
  using e3::kBatchRows;
  const int n = c->n;
  for (int g0 = 0; g0 < n_seq; g0 += kBatchRows) {
    const int gn = std::min(kBatchRows, n_seq - g0);
    std::vector<int> rows;
    for (int b = g0; b < g0 + gn; ++b) {
      const int ge = geff[size_t(b)];
      if (ge < gamma)
        E3_HIP(c, e3::launch_fill_i32(out + size_t(b) * gamma + ge, -1, gamma - ge, s), "fill");
      if (ge > 0) rows.push_back(b);
    }
    if (rows.empty()) continue;
    std::stable_sort(rows.begin(), rows.end(),
                     [&](int x, int y) { return geff[size_t(x)] > geff[size_t(y)]; });
    e3::BatchRows br{};
    br.m = int(rows.size());
    for (int r = 0; r < br.m; ++r) {
      const int b = rows[size_t(r)];
      br.orig[r] = b;
      br.slot[r] = seq_ids[b];
      br.pos0[r] = c->ledger.seq(seq_ids[b]).committed;
      br.row0[r] = local ? 0 : br.pos0[r];
      br.geff[r] = geff[size_t(b)];
    }
    auto gemm = [&](const uint16_t* W, int N, int K, const uint16_t* xh, const uint16_t* xl, int ldx,
                    int m, const e3::BGemmPlan& p, int epi) {
      e3::BGemmArgs ga{};
      ga.W = W; ga.N = N; ga.K = K; ga.Xhi = xh; ga.Xlo = xl; ga.ldx = ldx; ga.m = m;
      ga.P = c->b_P;
      ga.act_hi = c->bx_b_hi; ga.act_lo = c->bx_b_lo; ga.ld_act = c->bld_b;
      ga.cand_v = c->b_cand_v; ga.cand_i = c->b_cand_i; ga.ncand = c->b_ncand;
      ga.logits = (dbg && dbg->logits) ? c->b_logits : nullptr;
      return e3::launch_bgemm(ga, p, epi, s);
    };
    // a projection into the split-K partials b_P [splits][32][N]: the LDS-tiled GEMM
    // over all 32 activation rows (rows past m are never read back), else the
    // fragment-load GEMM; *S receives the split count
    auto proj = [&](const uint16_t* W, const uint16_t* Wt, int N, int K, const uint16_t* xh,
                    const uint16_t* xl, int ldx, int m, const e3::GemmPlan& tp, const e3::BGemmPlan& bp,
                    int* S) {
      if (tp.splits) {  // the skinny GEMM over the step-tiled copy
        *S = tp.splits;
        return e3::launch_gemm_tiled(xh, xl, ldx, Wt, c->b_P, kBatchRows, N, K, tp, s);
      }
      *S = bp.splits;
      return gemm(W, N, K, xh, xl, ldx, m, bp, e3::kBEpiPartial);
    };
    int S_enc = 0;
    if (!stored) {
      ProfScope ps(c, 6, s);
      E3_HIP(c, e3::launch_bpack_aux(br, a0, a1, a2, n, c->bx_a_hi, c->bx_a_lo, c->bld_a, s), "pack");
      E3_HIP(c, proj(c->w_fc, c->bt_enc, n, 3 * n, c->bx_a_hi, c->bx_a_lo, c->bld_a, br.m, c->tp_enc,
                     c->bp_enc, &S_enc), "encode");
    }
    const int steps = br.geff[0];
    for (int j = 0; j < steps; ++j) {
      int m = 0;
      while (m < br.m && br.geff[m] > j) ++m;
      e3::BPrepArgs pa{};
      pa.br = br; pa.m = m; pa.step = j; pa.gamma = gamma; pa.boundary_tok = btok;
      pa.cand_v = c->b_cand_v; pa.cand_i = c->b_cand_i; pa.ncand = c->b_ncand;
      pa.d2t = c->d2t; pa.dv = c->dv; pa.out_ids = out; pa.embed = c->embed; pa.vocab = c->vt;
      pa.n = n; pa.w_in = c->nrm_in; pa.w_hid = c->nrm_hid; pa.eps = c->cfg.rms_eps;
      pa.G = c->b_G; pa.Penc = c->b_P; pa.S_enc = S_enc;
      pa.bnd = stored ? c->bnd_y : nullptr;
      pa.Xhi = c->bx_a_hi; pa.Xlo = c->bx_a_lo; pa.ldx = c->bld_a;
      pa.dbg_hidden = dbg ? dbg->hidden : nullptr;
      pa.status = c->status;
      const int Nqkv = c->qd + 2 * c->kvd;
      {
        ProfScope ps(c, 2, s);
        E3_HIP(c, e3::launch_bprep(pa, s), "prep");
        int S_qkv = 0;
        E3_HIP(c, proj(c->w_qkv, c->bt_qkv, Nqkv, 2 * n, c->bx_a_hi, c->bx_a_lo, c->bld_a, m, c->tp_qkv,
                       c->bp_qkv, &S_qkv), "qkv");
        e3::BQkvArgs qa{};
        qa.P = c->b_P; qa.S = S_qkv; qa.N = Nqkv; qa.br = br; qa.m = m; qa.step = j;
        qa.n_head = c->nh; qa.n_head_kv = c->nkv; qa.head_dim = c->hd; qa.rope_dim = c->rot;
        qa.inv_freq = c->inv_freq; qa.q = c->b_q;
        qa.kv = local ? c->kv_local : c->kv;
        qa.seq_elems = local ? c->kv_local_elems : c->kv_seq_elems;
        qa.kv_f32 = c->kv_f32; qa.cap = local ? c->cap_local : c->cap;
        E3_HIP(c, e3::launch_bqkv(qa, s), "qkv rows");
      }
      {
        e3::AttnArgs aa{};
        aa.q = c->b_q; aa.kv_f32 = c->kv_f32;
        aa.k_cache = local ? c->k_local(0) : c->k_of(0);
        aa.v_cache = local ? c->v_local(0) : c->v_of(0);
        aa.cap = local ? c->cap_local : c->cap;
        aa.n_head = c->nh; aa.n_head_kv = c->nkv; aa.head_dim = c->hd;
        aa.part_o = c->b_po; aa.part_ml = c->b_pml; aa.batched = 1; aa.step = j;
        aa.seq_elems = local ? c->kv_local_elems : c->kv_seq_elems; aa.br = br;
        ProfScope ps(c, 5, s);
        E3_HIP(c, e3::launch_attn_batched(aa, m, c->bx_b_hi, c->bx_b_lo, c->bld_b, s), "attention");
      }
      {
        ProfScope ps(c, 4, s);
        int S_o = 0;
        E3_HIP(c, proj(c->w_o, c->bt_o, n, c->qd, c->bx_b_hi, c->bx_b_lo, c->bld_b, m, c->tp_o, c->bp_o,
                       &S_o), "o_proj");
        e3::BResidArgs ra{};
        ra.P = c->b_P; ra.S = S_o; ra.n = n; ra.m = m; ra.resid = c->b_G; ra.y = c->b_X1;
        ra.eps = c->cfg.rms_eps; ra.w1 = c->nrm_post; ra.x1_hi = c->bx_z_hi; ra.x1_lo = c->bx_z_lo;
        ra.ld1 = n; ra.br = br; ra.step = j; ra.gamma = gamma;
        E3_HIP(c, e3::launch_bresid(ra, s), "o_proj rows");
      }
      {
        ProfScope ps(c, 1, s);
        if (c->tp_gu.splits == 1) {
          e3::BGemmArgs ga{};
          ga.W = c->bt_gu; ga.tiled = 1; ga.N = 2 * c->ff; ga.K = n; ga.Xhi = c->bx_z_hi; ga.Xlo = c->bx_z_lo;
          ga.ldx = n; ga.m = m;
          ga.act_hi = c->bx_b_hi; ga.act_lo = c->bx_b_lo; ga.ld_act = c->bld_b;
          E3_HIP(c, e3::launch_sgemm_fused(ga, e3::kBEpiSilu, s), "gate/up");
        } else if (c->tp_gu.splits) {
          E3_HIP(c, e3::launch_gemm_tiled(c->bx_z_hi, c->bx_z_lo, n, c->bt_gu, c->b_P, kBatchRows,
                                          2 * c->ff, n, c->tp_gu, s), "gate/up");
          E3_HIP(c, e3::launch_bact(c->b_P, c->tp_gu.splits, c->ff, m, c->bx_b_hi, c->bx_b_lo,
                                    c->bld_b, s), "silu");
        } else {
          E3_HIP(c, gemm(c->w_gu, 2 * c->ff, n, c->bx_z_hi, c->bx_z_lo, n, m, c->bp_gu,
                         e3::kBEpiSilu), "gate/up");
        }
      }
      {
        ProfScope ps(c, 3, s);
        int S_d = 0;
        E3_HIP(c, proj(c->w_d, c->bt_d, n, c->ff, c->bx_b_hi, c->bx_b_lo, c->bld_b, m, c->tp_d, c->bp_d,
                       &S_d), "down");
        // g_next; RMSNorm(g_next, norm) for the lm_head and RMSNorm(g_next, hidden_norm)
        // as the second half of the next step's QKV input
        e3::BResidArgs ra{};
        ra.P = c->b_P; ra.S = S_d; ra.n = n; ra.m = m; ra.resid = c->b_X1; ra.y = c->b_G;
        ra.eps = c->cfg.rms_eps;
        ra.w1 = c->nrm_fin; ra.x1_hi = c->bx_h_hi; ra.x1_lo = c->bx_h_lo; ra.ld1 = n;
        ra.w2 = c->nrm_hid; ra.x2_hi = c->bx_a_hi + n; ra.x2_lo = c->bx_a_lo + n; ra.ld2 = c->bld_a;
        ra.br = br; ra.step = j; ra.gamma = gamma;
        ra.dbg_hidden = dbg ? dbg->hidden : nullptr;
        E3_HIP(c, e3::launch_bresid(ra, s), "down rows");
      }
      {
        ProfScope ps(c, 0, s);
        if (c->tp_lm.splits == 1) {
          e3::BGemmArgs ga{};
          ga.W = c->bt_lm; ga.tiled = 1; ga.N = c->dv; ga.K = n; ga.Xhi = c->bx_h_hi; ga.Xlo = c->bx_h_lo;
          ga.ldx = n; ga.m = m;
          ga.cand_v = c->b_cand_v; ga.cand_i = c->b_cand_i; ga.ncand = c->b_ncand;
          ga.logits = (dbg && dbg->logits) ? c->b_logits : nullptr;
          E3_HIP(c, e3::launch_sgemm_fused(ga, e3::kBEpiArgmax, s), "lm_head");
        } else if (c->tp_lm.splits) {
          E3_HIP(c, e3::launch_gemm_tiled(c->bx_h_hi, c->bx_h_lo, n, c->bt_lm, c->b_P, kBatchRows,
                                          c->dv, n, c->tp_lm, s), "lm_head");
          E3_HIP(c, e3::launch_bcand(c->b_P, c->tp_lm.splits, c->dv, m, c->b_cand_v, c->b_cand_i,
                                     (dbg && dbg->logits) ? c->b_logits : nullptr, s),
                 "lm_head candidates");
        } else {
          E3_HIP(c, gemm(c->w_lm, c->dv, n, c->bx_h_hi, c->bx_h_lo, n, m, c->bp_lm,
                         e3::kBEpiArgmax), "lm_head");
        }
      }
      if (dbg && dbg->logits)
        for (int r = 0; r < m; ++r)
          E3_HIP(c, hipMemcpyAsync(dbg->logits + (size_t(br.orig[r]) * gamma + j) * c->dv,
                                   c->b_logits + size_t(r) * c->dv, size_t(c->dv) * 4,
                                   hipMemcpyDeviceToDevice, s), "dbg logits");
    }
    E3_HIP(c, e3::launch_bfinal(c->status, br, br.m, gamma, c->b_cand_v, c->b_cand_i, c->b_ncand, c->d2t,
                                c->dv, out, s), "argmax");
  }
  return EAGLE3_OK;
}

}  // namespace

extern "C" {

int eagle3_draft_chain(eagle3_ctx* ctx, int32_t n_seq, const int32_t* seq_ids_host,
                       const int32_t* boundary_tok_dev, const float* aux0_dev,
                       const float* aux1_dev, const float* aux2_dev, int32_t gamma,
                       uint32_t flags, int32_t* out_ids_dev, int32_t* gamma_eff_host,
                       const eagle3_debug* dbg, void* stream) {
  if (!ctx) return EAGLE3_E_INVAL;
  if (n_seq < 0 || (n_seq > 0 && (!seq_ids_host || !gamma_eff_host)))
    return set_err(ctx, EAGLE3_E_INVAL, "bad sequence list");
  if (flags & ~(EAGLE3_KEEP_SPEC | EAGLE3_STORED_BOUNDARY | EAGLE3_ROUND_LOCAL))
    return set_err(ctx, EAGLE3_E_INVAL, "unknown flag");
  const bool local = (flags & EAGLE3_ROUND_LOCAL) != 0;
  if (local && (flags & EAGLE3_KEEP_SPEC))
    return set_err(ctx, EAGLE3_E_INVAL, "a round-local chain keeps no speculative rows");
  if (n_seq == 0) return EAGLE3_OK;
  const bool stored = (flags & EAGLE3_STORED_BOUNDARY) != 0;
  if (!boundary_tok_dev || (gamma > 0 && !out_ids_dev))
    return set_err(ctx, EAGLE3_E_INVAL, "null input pointer");
  if (stored) {
    if (aux0_dev || aux1_dev || aux2_dev)
      return set_err(ctx, EAGLE3_E_INVAL, "taps given with EAGLE3_STORED_BOUNDARY");
  } else {
    if (!aux0_dev || !aux1_dev || !aux2_dev) return set_err(ctx, EAGLE3_E_INVAL, "null input pointer");
    if (!aligned16(aux0_dev) || !aligned16(aux1_dev) || !aligned16(aux2_dev))
      return set_err(ctx, EAGLE3_E_INVAL, "tap pointers must be 16-byte aligned");
  }
  std::vector<int32_t> geff((size_t)n_seq);
  for (int b = 0; b < n_seq; ++b) {
    const char* why = nullptr;
    const int s = seq_ids_host[b];
    int rc = ctx->ledger.admit_chain(s, gamma, stored, local, &geff[size_t(b)], &why);
    if (rc) return set_err(ctx, rc, why);
    for (int j = 0; j < b; ++j)
      if (seq_ids_host[j] == s) return set_err(ctx, EAGLE3_E_INVAL, "duplicate sequence id");
  }
  for (int b = 0; b < n_seq; ++b) gamma_eff_host[b] = geff[size_t(b)];

  hipStream_t s = as_stream(stream);
  const int n = ctx->n;
  if (n_seq > 1) {
    const int rc = draft_chain_batched(ctx, n_seq, seq_ids_host, boundary_tok_dev, aux0_dev,
                                       aux1_dev, aux2_dev, stored, local, gamma, out_ids_dev, geff,
                                       dbg, s);
    if (rc) return rc;
    if (!local)
      for (int b = 0; b < n_seq; ++b)
        ctx->ledger.do_chain(seq_ids_host[b], geff[size_t(b)], (flags & EAGLE3_KEEP_SPEC) != 0);
    return EAGLE3_OK;
  }
  for (int b = 0; b < n_seq; ++b) {
    const int sq = seq_ids_host[b];
    const int L = ctx->ledger.seq(sq).committed;
    const int ge = geff[size_t(b)];
    int32_t* out_b = out_ids_dev + size_t(b) * gamma;
    if (ge < gamma) E3_HIP(ctx, e3::launch_fill_i32(out_b + ge, -1, gamma - ge, s), "fill");
    if (ge == 0) continue;
    // the first step's g: the stored boundary feature of the sequence, or the
    // encode of the given taps
    eagle3_ctx::GBuf g_bnd;
    if (stored) {
      g_bnd.y = ctx->bnd_y + size_t(sq) * n;
      g_bnd.w_hid = ctx->bnd_w + size_t(sq) * n;
      g_bnd.ssq = ctx->bnd_ssq + sq;
      g_bnd.count = 1;
    } else {
      e3::VecOut eo{ctx->gb[0].y, ctx->gb[0].w_hid, ctx->nrm_hid, nullptr, nullptr, ctx->gb[0].ssq};
      ProfScope ps(ctx, 6, s, true);
      E3_HIP(ctx, e3::launch_encode(ctx->wq(ctx->w_fc, ctx->i4_fc), ctx->ws(ctx->i4_fc), n,
                                    aux0_dev + size_t(b) * n, aux1_dev + size_t(b) * n,
                                    aux2_dev + size_t(b) * n, eo, ctx->gcfg[e3::kGemvEncode], s),
             "encode");
    }
    const eagle3_ctx::GBuf* g = stored ? &g_bnd : &ctx->gb[0];
    // the first step's hidden-half sums, when the append that stored the boundary
    // feature computed them
    const float* hsum0 = (stored && ctx->defer_qkv && ctx->bnd_hsum && ctx->bnd_hsum_ok[size_t(sq)])
                             ? ctx->bnd_hsum + size_t(sq) * ((ctx->nh + 2 * ctx->nkv) * ctx->hd)
                             : nullptr;
    if (dbg && dbg->hidden)
      E3_HIP(ctx, hipMemcpyAsync(dbg->hidden + size_t(b) * (gamma + 1) * n, g->y,
                                 size_t(n) * 4, hipMemcpyDeviceToDevice, s), "dbg hidden");
    for (int j = 0; j < ge; ++j) {
      const int pos = L + j;
      const int row = local ? j : pos;  // KV row written (and rows 0..row attended)
      void* kc = local ? ctx->k_local(sq) : ctx->k_of(sq);
      void* vc = local ? ctx->v_local(sq) : ctx->v_of(sq);
      const int cap = local ? ctx->cap_local : ctx->cap;
      const eagle3_ctx::GBuf* gn = &ctx->gb[1 + (j & 1)];
      e3::QkvArgs qa{};
      qa.w_qkv = ctx->wq(ctx->w_qkv, ctx->i4_qkv); qa.s_qkv = ctx->ws(ctx->i4_qkv); qa.n = n; qa.n_head = ctx->nh; qa.n_head_kv = ctx->nkv;
      qa.head_dim = ctx->hd; qa.rope_dim = ctx->rot; qa.inv_freq = ctx->inv_freq;
      qa.eps = ctx->cfg.rms_eps; qa.embed = ctx->embed; qa.vocab = ctx->vt; qa.status = ctx->status;
      if (j == 0) {
        qa.tok = boundary_tok_dev + b;
        qa.prev_count = 0;
      } else {
        qa.prev_val = ctx->lm_pv; qa.prev_idx = ctx->lm_pi; qa.prev_count = ctx->lm_grid;
        qa.d2t = ctx->d2t; qa.dv = ctx->dv; qa.prev_tok = ctx->lm_pt;
        qa.prev_out_id = out_b + (j - 1); qa.tok_store = ctx->tok_slots + (j - 1);
      }
      qa.gw = g->w_hid; qa.g_ssq = g->ssq; qa.g_ssq_count = g->count;
      qa.w_in = ctx->nrm_in; qa.pos = pos; qa.row = row; qa.q_out = ctx->q;
      qa.tok_tab = ctx->tok_tab; qa.w_hid_rows = ctx->w_qkv_h;
      qa.k_cache = kc; qa.v_cache = vc; qa.cap = cap;
      qa.kv_f32 = ctx->kv_f32;
      if (ctx->kv_q) {  // the new row goes to the fp32 stage; attention quantizes it
        qa.k_cache = ctx->kv_stage; qa.v_cache = ctx->kv_stage + ctx->kvd;
        qa.cap = 1; qa.row = 0; qa.kv_f32 = 1;
      }
      const int N_qkv = (ctx->nh + 2 * ctx->nkv) * ctx->hd;
      if (!ctx->defer_qkv) {
        ProfScope ps(ctx, 2, s, true);
        E3_HIP(ctx, e3::launch_qkv(qa, ctx->gcfg[e3::kGemvQkv], s), "qkv");
      } else if (j == 0 && !hsum0) {
        // deferred QKV: the first step's hidden half alone (later steps' run in the
        // lm_head launch of the step before); the attention kernel finishes the step
        const e3::QhArgs qh = ctx->qh_args(*g);
        e3::LmHeadArgs none{};
        ProfScope ps(ctx, 2, s, true);
        E3_HIP(ctx, e3::launch_lmhead_qh(none, qh, ctx->gcfg[e3::kGemvLmHead], s), "qkv hidden half");
      }
      e3::AttnArgs aa{};
      aa.q = ctx->q; aa.k_cache = kc; aa.v_cache = vc; aa.cap = cap;
      aa.kv_f32 = ctx->kv_f32;
      aa.kv_q = ctx->kv_q; aa.kv_new = ctx->kv_q ? ctx->kv_stage : nullptr;
      aa.T = row + 1; aa.n_head = ctx->nh; aa.n_head_kv = ctx->nkv; aa.head_dim = ctx->hd;
      aa.part_o = ctx->part_o; aa.part_ml = ctx->part_ml; aa.out = ctx->ao;
      if (ctx->defer_qkv) {
        aa.dq = 1;
        aa.dq_hsum = (j == 0 && hsum0) ? hsum0 : ctx->hsum;
        aa.dqa = qa;
      }
      {
        ProfScope ps(ctx, 5, s);
        E3_HIP(ctx, e3::launch_attn(aa, s), "attention");
      }
      {
        e3::VecOut oo{ctx->x1, ctx->x1w, ctx->nrm_post, nullptr, nullptr, ctx->x1_ssq};
        ProfScope ps(ctx, 4, s, true);
        E3_HIP(ctx, e3::launch_gemv_resid(ctx->wq(ctx->w_o, ctx->i4_o), ctx->ws(ctx->i4_o), n, ctx->qd,
                                          ctx->ao, g->y, oo,
                                          ctx->gcfg[e3::kGemvO], s), "o_proj");
      }
      {
        ProfScope ps(ctx, 1, s, true);
        E3_HIP(ctx, e3::launch_gateup(ctx->wq(ctx->w_gu, ctx->i4_gu), ctx->ws(ctx->i4_gu), ctx->ff, n,
                                      ctx->x1w, ctx->x1_ssq, ctx->x1_count,
                                      ctx->cfg.rms_eps, ctx->act, ctx->gcfg[e3::kGemvGateUp], s),
               "gate/up");
      }
      {
        e3::VecOut dn{gn->y, gn->w_norm, ctx->nrm_fin, gn->w_hid, ctx->nrm_hid, gn->ssq};
        ProfScope ps(ctx, 3, s, true);
        E3_HIP(ctx, e3::launch_gemv_resid(ctx->wq(ctx->w_d, ctx->i4_d), ctx->ws(ctx->i4_d), n, ctx->ff,
                                          ctx->act, ctx->x1, dn,
                                          ctx->gcfg[e3::kGemvDown], s), "down");
      }
      e3::LmHeadArgs la{};
      la.w_lm = ctx->wq(ctx->w_lm, ctx->i4_lm); la.s_lm = ctx->ws(ctx->i4_lm); la.dv = ctx->dv; la.n = n; la.hw = gn->w_norm; la.h_ssq = gn->ssq;
      la.h_ssq_count = gn->count; la.eps = ctx->cfg.rms_eps;
      la.logits_dbg = (dbg && dbg->logits) ? dbg->logits + (size_t(b) * gamma + j) * ctx->dv : nullptr;
      la.part_val = ctx->lm_pv; la.part_idx = ctx->lm_pi;
      la.d2t = ctx->d2t; la.part_tok = ctx->lm_pt;
      if (ctx->defer_qkv && j + 1 < ge) {  // with the next step's hidden-half QKV
        const e3::QhArgs qh = ctx->qh_args(*gn);
        ProfScope ps(ctx, 9, s, true);
        E3_HIP(ctx, e3::launch_lmhead_qh(la, qh, ctx->gcfg[e3::kGemvLmHead], s), "lm_head + qkv hidden half");
      } else {
        ProfScope ps(ctx, 0, s, true);
        E3_HIP(ctx, e3::launch_lmhead(la, ctx->gcfg[e3::kGemvLmHead], s), "lm_head");
      }
      if (dbg && dbg->hidden)
        E3_HIP(ctx, hipMemcpyAsync(dbg->hidden + (size_t(b) * (gamma + 1) + j + 1) * n, gn->y,
                                   size_t(n) * 4, hipMemcpyDeviceToDevice, s), "dbg hidden");
      g = gn;
    }
    E3_HIP(ctx, e3::launch_argmax_finalize(ctx->status, ctx->lm_pv, ctx->lm_pi, ctx->lm_pt, ctx->lm_grid, ctx->d2t,
                                           ctx->dv, out_b + (ge - 1), ctx->tok_slots + (ge - 1), s),
           "argmax");
  }
  if (!local)
    for (int b = 0; b < n_seq; ++b)
      ctx->ledger.do_chain(seq_ids_host[b], geff[size_t(b)], (flags & EAGLE3_KEEP_SPEC) != 0);
  return EAGLE3_OK;
}

int eagle3_profile_enable(eagle3_ctx* ctx, int32_t kernel, int32_t enable) {
  if (!ctx) return EAGLE3_E_INVAL;
  if (kernel < 0 || kernel >= kProfKernels) return set_err(ctx, EAGLE3_E_INVAL, "bad kernel id");
  if (!enable) { ctx->prof.kernel = -1; return EAGLE3_OK; }
  const size_t want = 2 * 8192;
  while (ctx->prof.ev.size() < want) {
    hipEvent_t e;
    E3_HIP(ctx, hipEventCreate(&e), "hipEventCreate");
    ctx->prof.ev.push_back(e);
  }
  ctx->prof.kernel = kernel;
  ctx->prof.used = 0;
  return EAGLE3_OK;
}

int eagle3_profile_read(eagle3_ctx* ctx, double* total_ms, int64_t* launches) {
  if (!ctx || !total_ms || !launches) return EAGLE3_E_INVAL;
  double tot = 0.0;
  for (size_t i = 0; i + 1 < ctx->prof.used; i += 2) {
    E3_HIP(ctx, hipEventSynchronize(ctx->prof.ev[i + 1]), "event sync");
    float ms = 0.f;
    E3_HIP(ctx, hipEventElapsedTime(&ms, ctx->prof.ev[i], ctx->prof.ev[i + 1]), "elapsed");
    tot += ms;
  }
  *total_ms = tot;
  *launches = int64_t(ctx->prof.used / 2);
  return EAGLE3_OK;
}

void eagle3_test_fail_allocation(int32_t n) { e3::g_alloc_fault.store(n > 0 ? n : 0); }

int64_t eagle3_test_live_allocations(void) { return e3::g_live_allocs.load(); }

// ---- the ledger on its own ----------------------------------------------------
int eagle3_ledger_create(int32_t max_ctx, int32_t max_seqs, int32_t max_gamma, eagle3_ledger** out) {
  if (!out) return EAGLE3_E_INVAL;
  *out = nullptr;
  if (max_ctx < 1 || max_seqs < 1 || max_gamma < 1) return EAGLE3_E_INVAL;
  eagle3_ledger* l = new (std::nothrow) eagle3_ledger();
  if (!l) return EAGLE3_E_OOM;
  l->l = e3::Ledger(max_ctx, max_seqs, max_gamma);
  *out = l;
  return EAGLE3_OK;
}

void eagle3_ledger_destroy(eagle3_ledger* l) { delete l; }

int eagle3_ledger_prefill(eagle3_ledger* l, int32_t seq, int32_t T, int32_t with_boundary) {
  if (!l) return EAGLE3_E_INVAL;
  int rc = l->l.check_prefill(seq, T, nullptr);
  if (rc) return rc;
  if (T == 0 && !with_boundary) return EAGLE3_OK;
  l->l.do_prefill(seq, T, with_boundary != 0);
  return EAGLE3_OK;
}

int eagle3_ledger_chain(eagle3_ledger* l, int32_t seq, int32_t gamma, uint32_t flags,
                        int32_t* gamma_eff) {
  if (!l || !gamma_eff) return EAGLE3_E_INVAL;
  if (flags & ~(EAGLE3_KEEP_SPEC | EAGLE3_STORED_BOUNDARY | EAGLE3_ROUND_LOCAL))
    return EAGLE3_E_INVAL;
  const bool local = (flags & EAGLE3_ROUND_LOCAL) != 0;
  if (local && (flags & EAGLE3_KEEP_SPEC)) return EAGLE3_E_INVAL;
  int32_t g = 0;
  int rc = l->l.admit_chain(seq, gamma, (flags & EAGLE3_STORED_BOUNDARY) != 0, local, &g, nullptr);
  if (rc) return rc;
  if (!local) l->l.do_chain(seq, g, (flags & EAGLE3_KEEP_SPEC) != 0);
  *gamma_eff = g;
  return EAGLE3_OK;
}

int eagle3_ledger_rebuild(eagle3_ledger* l, int32_t seq, int32_t n_accepted, int32_t with_boundary) {
  if (!l) return EAGLE3_E_INVAL;
  int rc = l->l.check_rebuild(seq, n_accepted, nullptr);
  if (rc) return rc;
  l->l.do_rebuild(seq, n_accepted, with_boundary != 0);
  return EAGLE3_OK;
}

int eagle3_ledger_rewind(eagle3_ledger* l, int32_t seq, int32_t new_len) {
  if (!l) return EAGLE3_E_INVAL;
  int rc = l->l.check_rewind(seq, new_len, nullptr);
  if (rc) return rc;
  l->l.do_rewind(seq, new_len);
  return EAGLE3_OK;
}

int eagle3_ledger_len(const eagle3_ledger* l, int32_t seq, int32_t* committed, int32_t* spec) {
  if (!l || !committed || !spec) return EAGLE3_E_INVAL;
  if (!l->l.valid_seq(seq)) return EAGLE3_E_INVAL;
  *committed = l->l.seq(seq).committed;
  *spec = l->l.seq(seq).spec;
  return EAGLE3_OK;
}

}  // extern "C"
