// Host-side launchers of the gfx950 kernels (one translation unit per family).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace e3 {

// Kernel-accurate timing of one launch for measurement: when armed, the next GEMV
// launch of the calling thread goes through hipExtLaunchKernelGGL with these
// events, which record the kernel's own start and end (no extra queue packets).
// Device status word of a drafter handle: bits raised by kernels that meet bad
// device-side inputs (the kernel still reads in bounds: an out-of-range id reads the
// nearest valid row, an argmax over NaN logits takes draft id 0).
constexpr uint32_t kStatusBadToken = 1u;   // a token id outside [0, target_vocab)
constexpr uint32_t kStatusNanLogits = 2u;  // a draft step whose logits were all NaN
constexpr uint32_t kStatusAppendRange = 4u;  // a teacher-forced fp16 activation out of range

// Fault injection for tests (include/eagle3_testing.h): while positive, every
// device allocation of the library counts it down and the one that brings it to
// zero fails as out of memory.
bool alloc_fault_fires();
// count of the device and pinned host allocations the library holds (all handles)
void note_alloc();
void note_free(size_t n);

struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool armed = false;
};
inline thread_local LaunchEvents g_launch_ev;


// ---- GEMV family (bf16 weights, fp32 activations and accumulate) ----
// `cfg` selects a launch configuration from E3_GEMV_CONFIGS (gemv_cfg.hpp).

// Output of a GEMV whose result y feeds an RMSNorm downstream: y itself, y
// weighted by up to two norm weights, and one partial sum of y^2 per block.
struct VecOut {
  float* y;
  float* yw1;          // y * w1 (or NULL)
  const float* w1;
  float* yw2;          // y * w2 (or NULL)
  const float* w2;
  float* ssq;          // [grid] (or NULL)
};
int gemv_grid(int N, int cfg);  // blocks (= partial sums) of a launch over N rows

// Weights of the GEMVs: bf16 rows [N][K], or (a non-null scale pointer S) int4 rows:
// codes [N][K / 2] bytes (element 2i in the low nibble, stored as q + 8, q in
// [-7, 7]) and one bf16 scale per group of 32 weights, [N][K / 32]; the weight is
// scale * q.  K must then be a multiple of 32.  launch_quant_i4 makes them from
// bf16 rows: scale = bf16(max|w| / 7), q = clamp(rint(w / scale), -7, 7), both
// divisions IEEE fp32.
hipError_t launch_quant_i4(const uint16_t* W, int rows, int K, uint8_t* Q, uint16_t* S,
                           hipStream_t s);
// The int4 matrix (Q, S) [rows][K] as bf16 (hi, lo) with hi + lo == scale * q exactly
// (the weights of the teacher-forced MFMA passes).
hipError_t launch_dequant_i4_split(const uint8_t* Q, const uint16_t* S, int rows, int K, uint16_t* hi,
                                   uint16_t* lo, hipStream_t s);

// g[r] = fc[r,:] . [aux0; aux1; aux2]
hipError_t launch_encode(const uint16_t* w_fc, const uint16_t* S, int n, const float* a0,
                         const float* a1, const float* a2, const VecOut& out, int cfg,
                         hipStream_t s);

// Fused: [finish the previous step's argmax] -> cat = [RMSNorm(E[tok]); RMSNorm(g)] ->
// (the hidden half arrives pre-weighted as gw = g * hidden_norm with the partial
// sums of g^2) ->
// q|k|v = W_qkv . cat (rows of q and k repacked so rotary partners are adjacent) ->
// NeoX rotation of q, k at `pos` -> q_out (fp32, natural order) and the K/V row `pos`
// of the cache (bf16, head-major).
struct QkvArgs {
  const uint16_t* w_qkv;
  const uint16_t* s_qkv;   // int4 scales (w_qkv then holds codes), or NULL
  int n, n_head, n_head_kv, head_dim, rope_dim;
  const double* inv_freq;  // [rope_dim / 2]: theta^(-2i / rope_dim)
  float eps;
  const uint16_t* embed;
  int vocab;               // rows of embed; an id outside [0, vocab) raises kStatusBadToken
  uint32_t* status;        // device status word
  const int32_t* tok;      // device: the token fed to this step (when prev_count == 0)
  // when prev_count > 0 the token is the argmax of the previous step's lm_head
  // candidates mapped through d2t; block 0 stores it to *prev_out_id and *tok_store
  const float* prev_val;
  const int32_t* prev_idx;
  int prev_count;
  const int32_t* d2t;
  int dv;
  const int32_t* prev_tok;  // [prev_count] target id of each candidate (i + d2t[i]), or NULL
  int32_t* prev_out_id;
  int32_t* tok_store;
  const float* gw;         // recurrent hidden times hidden_norm
  const float* g_ssq;      // per-block partial sums of g^2
  int g_ssq_count;
  const float* w_in;       // input_layernorm
  // optional token table: tok_tab[t][r] = W_qkv[r, :n] . (w_in * E[t]) / rms(E[t]) for
  // every row r of the repacked QKV matrix (the normalised embedding half); with it the
  // embedding half of W_qkv is not streamed
  const float* tok_tab;
  // with the table: the hidden half of W_qkv as its own contiguous [N][n] matrix (or
  // NULL: the rows' second halves are read in place, 2n apart)
  const uint16_t* w_hid_rows;
  int pos;                 // rotary position of the row
  int row;                 // KV row written (pos, or the step in a round-local scratch)
  float* q_out;
  void* k_cache;           // this sequence's [n_head_kv][cap][head_dim]
  void* v_cache;
  int cap;
  int kv_f32;              // cache element: fp32 (1) or bf16 (0)
};
hipError_t launch_qkv(const QkvArgs& a, int cfg, hipStream_t s);

// y[r] = W[r,:] . x + resid[r]   (o_proj, down_proj)
hipError_t launch_gemv_resid(const uint16_t* w, const uint16_t* S, int N, int K, const float* x,
                             const float* resid, const VecOut& out, int cfg, hipStream_t s);

// act[i] = silu(gate_i . z) * (up_i . z), z = xw / rms with xw = x1 * w_post and the
// rms from per-block partial sums of x1^2; W_gu rows interleaved
hipError_t launch_gateup(const uint16_t* w_gu, const uint16_t* S, int n_ff, int n, const float* xw,
                         const float* x_ssq, int ssq_count, float eps, float* act, int cfg,
                         hipStream_t s);

// logits = lm_head . (hw / rms) with hw = h * w_norm and the rms from per-block
// partial sums of h^2; each block stores its best (value, index) (lowest index on
// ties) and, when d2t is given, that index's target id i + d2t[i].  logits_dbg
// may be NULL.
struct LmHeadArgs {
  const uint16_t* w_lm;
  const uint16_t* s_lm;    // int4 scales (w_lm then holds codes), or NULL
  int dv, n;
  const float* hw;
  const float* h_ssq;
  int h_ssq_count;
  float eps;
  float* logits_dbg;
  float* part_val;         // [grid]
  int32_t* part_idx;       // [grid]
  const int32_t* d2t;      // [dv] or NULL
  int32_t* part_tok;       // [grid] (written when d2t is given)
};
int lmhead_grid(int dv, int cfg);
hipError_t launch_lmhead(const LmHeadArgs& a, int cfg, hipStream_t s);
// The recurrent half of the next draft step's QKV projection: it needs only that
// step's hidden state g, not its token, so it runs in the lm_head launch of the step
// before (or alone for a chain's first step): hsum[r] = W_qkv[r, n:2n] . gw / rms(g)
// for the N rows of the repacked QKV matrix, gw = g * hidden_norm.  The step's
// attention kernel adds the token table's row, rotates, and stores the K/V row
// (AttnArgs dq).
struct QhArgs {
  const uint16_t* w;      // bf16: row 0 of the hidden half (N rows of n values, ldw apart);
                          // int4: the codes of W_qkv (columns k0 .. k0 + n of N rows of ldw)
  const uint16_t* s;      // int4 scales (w then holds codes), or NULL
  size_t ldw;
  int k0;                 // int4: the hidden half's first column (n); bf16: 0
  int N, n;
  const float* gw;
  const float* g_ssq;     // per-block partial sums of g^2
  int g_ssq_count;
  float eps;
  float* hsum;            // [N]: W_qkv[r, n:2n] . gw / rms(g)
};
// lm_head as launch_lmhead (same configuration and candidate count) and hsum in one
// launch; with a.w_lm == NULL only hsum
hipError_t launch_lmhead_qh(const LmHeadArgs& a, const QhArgs& q, int cfg, hipStream_t s);
// the deferred-QKV attention reduces at most this many lm_head candidates (one batch
// per thread of its 256-thread blocks)
constexpr int kDqMaxCandidates = 2048;
// argmax over the candidates, target = i + d2t[i] (taken from pt when given)
// -> *out_id (and *tok_store if set)
hipError_t launch_argmax_finalize(uint32_t* status, const float* pv, const int32_t* pi, const int32_t* pt, int count,
                                  const int32_t* d2t, int dv, int32_t* out_id, int32_t* tok_store,
                                  hipStream_t s);

// A second set of tap streams for a teacher-forced pass: rows [rows_x, rows) of the
// pass read y[0..2] (row rows_x is y's row 0); rows_x >= rows means none.  Passed by
// value.
struct TapRowsB {
  const float* y[3];
  int rows_x;
};
inline TapRowsB no_tap_rows_b() { return TapRowsB{{nullptr, nullptr, nullptr}, 1 << 30}; }

// Multi-vector split-K GEMV for teacher-forced rows: P[z][m][r] (fp32) over K chunks z.
// Input: three fp32 streams x0|x1|x2 of row length seg concatenated along K (rows from
// yb.rows_x on taken from yb's streams), or (x1 == NULL) one fp32 matrix x0 [rows, K].
// rows <= 16; *splits_out receives the chunk count.
int gemv_multi_width(int rows);
int gemv_multi_splits(int rows, int N, int K);  // chunk count the launch will use
hipError_t launch_gemv_multi(const uint16_t* W, const uint16_t* S, int N, int K, const float* x0,
                             const float* x1, const float* x2, int seg, int rows, float* P,
                             int* splits_out, hipStream_t s, const TapRowsB& yb = no_tap_rows_b());
// launch_gemv_multi with one fp32 activation matrix x0 [rows, K], plus the hidden-half
// sums q (as launch_lmhead_qh without lm_head) in the same launch; S non-null: W
// holds int4 codes and S their scales, and q the int4 hidden half
hipError_t launch_gemv_multi_qh(const uint16_t* W, const uint16_t* S, int N, int K, const float* x0, int rows,
                                float* P, int* splits_out, const QhArgs& q, hipStream_t s);

// ---- batched drafting: up to kBatchRows sequences per pass ----
constexpr int kBatchRows = 32;
// The rows of one batched pass, ordered by admitted chain length (descending) so
// that the rows still drafting at step j are the prefix [0, m_j).  Passed by value.
struct BatchRows {
  int m;                      // rows in the pass
  int32_t orig[kBatchRows];   // row -> index in the caller's sequence list
  int32_t pos0[kBatchRows];   // committed rows = rotary position of step 0
  int32_t row0[kBatchRows];   // KV row of step 0: pos0, or 0 in a round-local scratch
  int32_t slot[kBatchRows];   // sequence id (draft-KV slot)
  int32_t geff[kBatchRows];   // admitted chain length (>= 1)
};

// ---- attention over the draft KV (split over context, LSE combine) ----
// ---- quantized draft KV (EAGLE3_KV_Q8Q5) ----
// A sequence's K region holds, in bytes: codes [nkv][cap][hd] (q8_0 code + 128), then
// fp16 scales [nkv][cap][hd / 32].  Its V region: code nibbles [nkv][cap][hd / 2], high
// bits [nkv][cap][hd / 8], then (D, M) fp16 pairs [nkv][cap][hd / 32] (one u32, D in
// the low half).  Within a row, with NB = hd / 32, dim 32 b + 16 h + c (c < 16) keeps
// its low 4 bits in nibble h of byte c NB + b and its bit 4 in bit (B % 4) + 4 h of
// high-bit byte B / 4, B = c NB + b (common.hpp vq_byte): an MFMA lane c reads its
// dims 16 t + c as one run of NB bytes.  Both regions are kvq_region_bytes long: 34
// bytes per 32 K values and 24 per 32 V values, as in the pages' block formats, with
// the V region padded to the K region's size rounded up to 256 bytes (so the V arrays
// start 16-byte aligned).
inline size_t kvq_region_bytes(int nkv, int cap, int hd) {
  return (size_t(nkv) * cap * (hd / 32) * 34 + 255) / 256 * 256;
}

struct AttnArgs {
  const float* q;          // [n_head * hd], roped
  const void* k_cache;     // [n_head_kv][cap][hd], fp32 or bf16 (or a quantized K region)
  const void* v_cache;
  int kv_f32;
  int kv_q;                // quantized regions (q8_0 K, q5_1 V)
  const float* kv_new;     // kv_q: the new row T - 1 in fp32, K [nkv][hd] then V; the
                           // block of its split quantizes it into the cache first
  int cap, T;              // rows 0..T-1 attended
  int n_head, n_head_kv, head_dim;
  float* part_o;           // [n_head][S][hd]
  float* part_ml;          // [n_head][S][2]
  float* out;              // [n_head * hd]
  // batched form (batched != 0): row r of blockIdx.z attends rows 0..row0[r]+step of
  // slot[r], whose K/V start seq_elems * slot elements past k_cache / v_cache; q and
  // the partials are per row ([row][n_head][hd], [row][n_head][S][...])
  int batched;
  int step;
  size_t seq_elems;
  BatchRows br;
  // deferred QKV (dq != 0; batch 1, fp32 or bf16 K/V): the step's q and its new K/V
  // row T - 1 are finished in this kernel from dq_hsum (QhArgs) and the token table
  // row of the step's token (dqa: token source, table, norms' partial sums, rotary
  // position, cache); q is then not read, and the block whose split holds row T - 1
  // stores the row and takes it into its softmax from LDS
  int dq;
  const float* dq_hsum;
  QkvArgs dqa;
};
int attn_max_splits(int cap, int head_dim, int n_head_kv);

// Verify-window attention: M query rows per head ([M][n_head][hd], roped), cache rows
// 0..ctx+M-1 ([n_head_kv][cap][hd], fp32 or bf16), query row m sees rows 0..ctx+m;
// out [M][n_head][hd].  Split partials go to part_o [M*n_head][S][hd] and part_ml
// [M*n_head][S][2] (attn_verify_workspace bytes in all, unused when S == 1).
struct VerifyArgs {
  const float* q;
  const void* k;
  const void* v;
  int kv_f32;
  int cap, ctx, M;
  int n_head, n_head_kv, head_dim;
  float* part_o;
  float* part_ml;
  float* out;
};
size_t attn_verify_workspace(int M, int n_head, int n_head_kv, int head_dim, int ctx, int kv_f32);
hipError_t launch_attn_verify(const VerifyArgs& a, size_t workspace_bytes, hipStream_t s);
// the allocation-free variant's device scratch (the current device's copy)
constexpr size_t kVerifyScratchBytes = size_t(16) << 20;
hipError_t verify_scratch_ptr(void** ptr);
// Splits the context, then (when more than one split) runs the combine kernel.
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
// Batched: split every row's context in chunks of one size, then combine per (row,
// head) into bf16 (hi, lo) pairs [row][ld] for the output projection.
int attn_batch_chunk(const BatchRows& br, int m, int step, int n_head_kv, int head_dim, int kv_f32);
int attn_batch_max_splits(int cap, int head_dim, int kv_f32);
hipError_t launch_attn_batched(const AttnArgs& a, int m, uint16_t* out_hi, uint16_t* out_lo, int ld,
                               hipStream_t s);

// ---- batched GEMMs on MFMA: Y[b][r] = sum_k X[b][k] W[r][k], b < m <= 32 ----
// X arrives as bf16 pairs (hi, lo = bf16(x - hi)) [32][ldx]; both are multiplied
// (two MFMAs per weight fragment), so the product carries ~16 mantissa bits of x.
enum BEpi { kBEpiPartial = 0, kBEpiSilu = 1, kBEpiArgmax = 2 };
struct BGemmArgs {
  const uint16_t* W;
  int N, K;
  const uint16_t* Xhi;
  const uint16_t* Xlo;
  int ldx, m;
  int kb;                  // K per split (set by the plan)
  float* P;                // kBEpiPartial: [splits][32][N]
  uint16_t* act_hi;        // kBEpiSilu: rows interleaved (gate_i, up_i) -> silu(gate) * up
  uint16_t* act_lo;        //   as a (hi, lo) pair [32][ld_act]
  int ld_act;
  float* cand_v;           // kBEpiArgmax: per (row b, block) best (value, index) [32][ncand]
  int32_t* cand_i;
  int ncand;
  float* logits;           // kBEpiArgmax, optional: [32][N]
  int tiled;               // W is the step-tiled copy (launch_tile_weights)
};
struct BGemmPlan {
  int variant, splits, kb, blocks;
};
BGemmPlan bgemm_plan(int N, int K, int epi);
hipError_t launch_bgemm(BGemmArgs a, const BGemmPlan& p, int epi, hipStream_t s);
// The skinny MFMA GEMM over the whole K (32 activation rows, split activations) with
// the kBEpiSilu or kBEpiArgmax epilogue of the arguments above; the argmax writes
// sgemm_tiles(N) candidates per row (ncand >= that).  K % 64 == 0.
int sgemm_tiles(int N);
hipError_t launch_sgemm_fused(const BGemmArgs& a, int epi, hipStream_t s);

// Row kernels of the batched step: one block of kBRowThreads per sequence row
// keeps the row in registers (up to kBRowMax values), so a row's sums, its RMS
// and the normalised (hi, lo) output take one pass.
constexpr int kBRowThreads = 1024;
constexpr int kBRowMax = 2 * 4 * kBRowThreads;

// X[r] = aux0|aux1|aux2 of caller row orig[r] (fp32 [n_seq][n] each) as (hi, lo)
hipError_t launch_bpack_aux(const BatchRows& br, const float* a0, const float* a1, const float* a2,
                            int n, uint16_t* Xhi, uint16_t* Xlo, int ldx, hipStream_t s);
// Start of step `step` for rows [0, m): the token (boundary token at step 0, else the
// argmax of the previous lm_head candidates through d2t, also stored to
// out_ids[orig * gamma + step - 1]), then X[r][0:n] = RMSNorm(E[tok], w_in) as
// (hi, lo).  At step 0 also g = sum of the encode partials (or, with bnd set, the
// stored boundary feature bnd[slot * n ..]) -> G and X[r][n:2n] = RMSNorm(g, w_hid)
// (later steps receive that half from the down projection's row kernel).
struct BPrepArgs {
  BatchRows br;
  int m, step, gamma;
  const int32_t* boundary_tok;
  const float* cand_v;
  const int32_t* cand_i;
  int ncand;
  const int32_t* d2t;
  int dv;
  int32_t* out_ids;
  const uint16_t* embed;
  int vocab, n;
  const float* w_in;
  const float* w_hid;
  float eps;
  float* G;                // [32][n]
  const float* Penc;       // step 0: encode partials [S][32][n]
  int S_enc;
  const float* bnd;        // step 0: stored boundary features [slots][n], or NULL
  uint16_t* Xhi;           // [32][ldx]
  uint16_t* Xlo;
  int ldx;
  float* dbg_hidden;       // optional [n_seq][gamma + 1][n]
  uint32_t* status;        // device status word
};
hipError_t launch_bprep(const BPrepArgs& a, hipStream_t s);
// q|k|v of rows [0, m) from the QKV partials: rotate q, k at pos0 + step; q -> [32][qd],
// k, v -> row row0 + step of each row's cache slot.
struct BQkvArgs {
  const float* P;
  int S, N;
  BatchRows br;
  int m, step;
  int n_head, n_head_kv, head_dim, rope_dim;
  const double* inv_freq;
  float* q;
  void* kv;                // cache of slot 0; slot s starts s * seq_elems elements later
  size_t seq_elems;
  int kv_f32, cap;
};
hipError_t launch_bqkv(const BQkvArgs& a, hipStream_t s);
// y = sum_z P[z] + resid (rows [0, m), width n) -> y, then RMSNorm(y, w1) and
// RMSNorm(y, w2) as (hi, lo) pairs (row strides ld1, ld2; the second may be NULL);
// optionally y -> dbg_hidden[orig][step + 1].
struct BResidArgs {
  const float* P;
  int S, n, m;
  const float* resid;
  float* y;
  float eps;
  const float* w1;
  uint16_t* x1_hi;
  uint16_t* x1_lo;
  int ld1;
  const float* w2;
  uint16_t* x2_hi;
  uint16_t* x2_lo;
  int ld2;
  BatchRows br;
  int step, gamma;
  float* dbg_hidden;
};
hipError_t launch_bresid(const BResidArgs& a, hipStream_t s);
// act = silu(sum_z P[z][2i]) * sum_z P[z][2i+1] as (hi, lo) [32][ld]
hipError_t launch_bact(const float* P, int S, int n_ff, int m, uint16_t* Xhi, uint16_t* Xlo, int ld,
                       hipStream_t s);
// lm_head candidates from split-K partials P[z][32][N]: for each row r < m and each
// block of kBCandCols columns, the best (value, index) of sum_z P[z][r][c] (the
// lowest index on ties) -> cand_v/cand_i[r * ncand + block]; the summed logits also
// to logits[r * N + c] when logits is not NULL.  ncand = bcand_count(N).
constexpr int kBCandCols = 2048;
inline int bcand_count(int N) { return (N + kBCandCols - 1) / kBCandCols; }
hipError_t launch_bcand(const float* P, int S, int N, int m, float* cand_v, int32_t* cand_i,
                        float* logits, hipStream_t s);
// rows [0, m): out_ids[orig * gamma + geff - 1] = d2t-mapped argmax of the candidates
hipError_t launch_bfinal(uint32_t* status, const BatchRows& br, int m, int gamma, const float* cand_v,
                         const int32_t* cand_i, int ncand, const int32_t* d2t, int dv,
                         int32_t* out_ids, hipStream_t s);

// ---- teacher-forced append (prefill / rebuild) ----
// A[t, 0:3n] = [aux0[t]; aux1[t]; aux2[t]] as bf16 (A_hi), rows from yb.rows_x on
// taken from yb's streams; with A_lo given, also the bf16 remainder
// A_lo = bf16(a - A_hi), so A_hi + A_lo carries ~16 mantissa bits.
// f16: the taps as fp16 (A_lo NULL; a value outside the fp16 range raises
// kStatusAppendRange), else bf16 (hi, lo) pairs (A_lo may be NULL: hi only)
hipError_t launch_pack_aux(const float* a0, const float* a1, const float* a2, int T, int n,
                           uint16_t* A_hi, uint16_t* A_lo, hipStream_t s,
                           const TapRowsB& yb = no_tap_rows_b(), int f16 = 0, uint32_t* status = nullptr);
// Boundary features of a teacher-forced pass: fc rows [T_cat, T_cat + count) are the
// next rounds' boundary rows; row T_cat + j goes to sequence slot slot[j]:
// y[slot] = f [n], yw[slot] = f * w_hid [n], ssq[slot] = sum f^2.
constexpr int kBndRows = 32;
struct BndOut {
  float* y;
  float* yw;
  float* ssq;
  int count;
  int32_t slot[kBndRows];
};
// cat[t] = [RMSNorm(E[tok[t]], w_in); RMSNorm(sum_z F[z][t], w_hid)] for t < T, F row
// stride n, split stride f_split (elements); written as fp32 (cat32) or as bf16
// (cat16, plus the bf16 remainder in cat16_lo when given).  Rows T .. T + bnd.count - 1
// of F are boundary rows, summed into bnd's slots.
hipError_t launch_tf_cat(uint32_t* status, const float* F, int splits, size_t f_split, int T, int n,
                         const uint16_t* embed, int vocab, const int32_t* tok, const float* w_in,
                         const float* w_hid, float eps, uint16_t* cat16, uint16_t* cat16_lo,
                         float* cat32, hipStream_t s, const BndOut* bnd = nullptr, float f_scale = 1.0f,
                         int f16 = 0);
// Up to kStoreSegs runs of consecutive rows of one append pass: rows
// [row0[s], row0[s + 1]) go to sequence slot[s] from position pos0[s] on.
constexpr int kStoreSegs = 32;
struct StoreSegs {
  int n;
  int32_t row0[kStoreSegs + 1];
  int32_t pos0[kStoreSegs];
  int32_t slot[kStoreSegs];
};
// every row t of the segments: kv = sum_z P[z][t] over [k(kvd) | v(kvd)] (k rows
// repacked, row stride 2*kvd, split stride p_split); rotate k at the row's position
// and store it into that cache row of its slot (slot s starts s * seq_elems
// elements past kv; K then V, each [n_head_kv][cap][head_dim]).
// (kv_q: quantized regions; seq_elems is then the bytes per slot, K region then V)
hipError_t launch_tf_store(const float* P, int splits, size_t p_split, const StoreSegs& segs,
                           int n_head_kv, int head_dim, int rope_dim, const double* inv_freq, void* kv,
                           size_t seq_elems, int cap, int kv_f32, hipStream_t s, int kv_q = 0,
                           float p_scale = 1.0f);
// rows [row0, row0 + nrows) of quantized K/V regions as fp32 [nrows][nkv][hd]
hipError_t launch_kvq_read(const void* kreg, const void* vreg, int nkv, int cap, int hd, int row0,
                           int nrows, float* k_out, float* v_out, hipStream_t s);

// C[z][M][N] (fp32) = (A_hi + A_lo)[M, kz-range] . B[N, kz-range]^T on bf16 MFMA
// (A_lo may be NULL: one product).  Row strides lda, ldb (elements); K split
// evenly over plan.splits.  The plan's tile width is 256 or 320 columns for
// 256-row tiles (M >= 256), 128 for 128-row tiles, and 128 weight rows per block
// for the skinny GEMM (M <= 32).
struct GemmPlan {
  int bn;      // output tile width
  int splits;  // K split (z planes of C)
};
GemmPlan gemm_plan(int M, int N, int K);
// f16: A and B hold fp16 values (one v_mfma_f32_16x16x32_f16 product, no A_lo)
hipError_t launch_gemm_bf16(const uint16_t* A_hi, const uint16_t* A_lo, int lda, const uint16_t* B,
                            int ldb, float* C, int M, int N, int K, const GemmPlan& plan,
                            hipStream_t s, bool f16 = false);
// The skinny GEMM's step-tiled weight copy: T [ceil(N / 128)][K / 64][128][64] of W
// [N][K] (K % 64 == 0; rows past N zero), tiled_weight_elems(N, K) elements; and the
// split-activation GEMM of up to 32 rows over it (C as launch_gemm_bf16's, plan from
// gemm_plan with bn 128)
size_t tiled_weight_elems(int N, int K);
hipError_t launch_tile_weights(const uint16_t* W, int N, int K, uint16_t* T, hipStream_t s);
hipError_t launch_gemm_tiled(const uint16_t* A_hi, const uint16_t* A_lo, int lda, const uint16_t* Bt, float* C,
                             int M, int N, int K, const GemmPlan& plan, hipStream_t s);
// the token table's build: ss[t] = sum E[t]^2; rows [r0, r0 + T) of w_in * E as bf16 (hi, lo)
hipError_t launch_tok_ss(const uint16_t* E, int vocab, int n, float* ss, hipStream_t s);
hipError_t launch_pack_embed(const uint16_t* E, const float* w_in, const float* ss, float eps, int r0, int T,
                             int n, uint16_t* A_hi, uint16_t* A_lo, hipStream_t s);
// dst[i] += src[i], i < count
hipError_t launch_add_f32(float* dst, const float* src, size_t count, hipStream_t s);
// dst[i] = fp16 bits of (bf16 src[i]) * 2^8, exact for 2^-25 <= |src| < 256 (and 0);
// any other weight raises kStatusAppendRange in *status
hipError_t launch_bf16_to_f16_x256(const uint16_t* src, uint16_t* dst, size_t count, uint32_t* status,
                                   hipStream_t s);

// ---- the synthetic target trunk (trunk.hip) ----
// status word bits raised by the trunk kernels
constexpr uint32_t kTrunkBadToken = 1u;   // an input id outside the vocabulary (row 0 read)
constexpr uint32_t kTrunkNanLogits = 2u;  // a row whose logits are all NaN (id 0 given)
struct TrunkLayer {
  const float *attn_norm, *mlp_norm;  // fp32 [n]
  const uint16_t *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;  // bf16 [out][in]
  float *k_cache, *v_cache;           // fp32 [nkv][cap][hd]
};
// scratch for up to max_tokens rows
struct TrunkBufs {
  float *x, *h, *z, *q, *k, *v, *o, *act, *logits;
  float *part_o, *part_ml;  // verify-attention split partials (ws_bytes in all)
  size_t ws_bytes;
};
struct TrunkArgs {
  int n, nh, nkv, hd, ff, vocab, n_layers, cap;
  float eps;
  const uint16_t* embed;      // bf16 [vocab][n]
  const float* final_norm;    // fp32 [n]
  const uint16_t* lm_head;    // bf16 [vocab][n]
  const double* inv_freq;     // [hd / 2]
  const TrunkLayer* layer;    // host array [n_layers]
  TrunkBufs buf;
  uint32_t* status;           // device status word
};
// one forward over T tokens at positions pos0 .. pos0 + T - 1: ids [T]; taps[j]
// [T][n] (or null): the residual stream entering the first layer, leaving layer
// n_layers / 2 - 1 and leaving the last layer
hipError_t launch_trunk_forward(const TrunkArgs& a, int T, int pos0, const int32_t* tok, int32_t* ids,
                                float* const taps[3], hipStream_t s);
// res = [a, bonus, status, drafts[0..g)]: a = longest prefix with drafts[i] ==
// verify[i], bonus = verify[a]; the status word is copied and cleared
hipError_t launch_accept(const int32_t* drafts, const int32_t* verify, int g, int32_t* res,
                         uint32_t* status, hipStream_t s);

// ---- load-time and bookkeeping helpers ----
// dst row dst_rows[i] = src row src_rows[i] (bf16 rows of row_len elements)
hipError_t launch_gather_rows(uint16_t* dst, const uint16_t* src, const int32_t* dst_rows,
                              const int32_t* src_rows, int count, int row_len, hipStream_t s);
hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t s);

}  // namespace e3
