/*
 * eagle3.h — C ABI of the MI355X (gfx950) EAGLE-3 drafter engine.
 *
 * The engine runs the EAGLE-3 draft head: an encoder `fc` over three captured
 * target hidden states, one Llama-style decoder layer with a persistent draft
 * KV cache, a draft-vocabulary lm_head, greedy argmax and the d2t map to target
 * ids.  Entry points follow the operations described in pegainfer PR #707
 * ("feat(eagle3): Qwen3 EAGLE-3 drafter forward pass (single-step + chain
 * rollout)", PR description: prefill, draft_chain / chain_round,
 * rebuild_after_verify) and the op sequence in the module doc of the
 * memra_engine 0.121.0 `eagle.rs` listing.
 *
 * Conventions (all entry points):
 *   - return int status: EAGLE3_OK (0) or a negative EAGLE3_E_* code;
 *     eagle3_last_error() gives a message for the last failing call;
 *   - every argument check runs before any device work is queued, so a
 *     failing call changes no state;
 *   - "dev" pointers are HIP device pointers, "host" pointers host memory;
 *     fp32 tap (aux) pointers must be 16-byte aligned (rows are read as vectors);
 *     inputs are borrowed for the call in stream order, outputs are written
 *     in stream order and are valid once the stream reaches the call;
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream);
 *   - one handle is used by one host thread at a time.
 */
#ifndef EAGLE3_H
#define EAGLE3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EAGLE3_OK = 0,
  EAGLE3_E_INVAL = -1,       /* bad argument (null pointer, id or count out of range) */
  EAGLE3_E_SHAPE = -2,       /* inconsistent tensor geometry */
  EAGLE3_E_UNSUPPORTED = -3, /* geometry the kernels do not handle */
  EAGLE3_E_CAPACITY = -4,    /* draft KV capacity exceeded */
  EAGLE3_E_STATE = -5,       /* call not allowed in the sequence's current state */
  EAGLE3_E_HIP = -6,         /* HIP runtime error */
  EAGLE3_E_OOM = -7          /* device allocation failed */
};

/* eagle3_draft_chain flag: keep the speculative rows (spec > 0) instead of
   rewinding at the end of the round; only eagle3_rewind clears them. */
#define EAGLE3_KEEP_SPEC 1u
/* eagle3_draft_chain flag: start each listed sequence from its stored boundary
   feature (set by eagle3_prefill / eagle3_rebuild_after_verify from next-boundary
   taps) instead of encoding taps; the tap pointers must then be NULL.  With the
   token table (and fp32 or bf16 K/V), an append pass of at most 16 rows that stores one
   boundary feature with teacher-forced rows also computes the hidden half of that
   feature's QKV projection (in its K/V launch), and the batch-1 chain that starts
   from it runs no launch of its own for it (environment EAGLE3_BOUNDARY_QH=0 turns
   this off).  Which launches a stored-boundary round issues thus depends on the
   append that stored the feature: a round captured in a graph replays the launches
   of its capture, so replay it only over the same stored feature. */
#define EAGLE3_STORED_BOUNDARY 2u
/* eagle3_draft_chain flag: the round-local drafter (memra_engine `eagle.rs`,
   `Eagle3Scratch`: the draft KV is a small scratch emptied every round).  Step j
   attends over the round's own rows 0..j only, held in a per-sequence scratch of
   max_gamma rows; rotary positions still continue from the committed length; the
   committed rows are neither read nor written, gamma_eff = gamma, and the call
   changes no length (a rebuild still needs a persistent chain round first).  Not
   combinable with EAGLE3_KEEP_SPEC. */
#define EAGLE3_ROUND_LOCAL 4u

typedef struct eagle3_ctx eagle3_ctx;

/* Drafter geometry (memra `Eagle3Draft` fields) plus capacity. */
typedef struct {
  int32_t n_embd;        /* hidden size n */
  int32_t n_head;        /* query heads */
  int32_t n_head_kv;     /* key/value heads; n_head % n_head_kv == 0 */
  int32_t head_dim;      /* 64, 128 or 256 */
  int32_t n_ff;          /* MLP width */
  int32_t draft_vocab;   /* rows of lm_head */
  int32_t target_vocab;  /* rows of the token embedding */
  int32_t n_aux;         /* captured taps; must be 3 */
  int32_t rope_dim;      /* rotated dims per head (even, <= head_dim); see eagle3_resolve_rope_dim */
  float rope_theta;
  float rms_eps;
  int32_t max_ctx;       /* admission bound per sequence; max_ctx + 1 rows are allocated */
  int32_t max_gamma;     /* largest chain length accepted */
  int32_t max_seqs;      /* sequence slots */
  int32_t kv_dtype;      /* EAGLE3_KV_F32 (default), EAGLE3_KV_BF16 or EAGLE3_KV_Q8Q5 */
  int32_t weight_format; /* EAGLE3_WEIGHTS_BF16 (default) or EAGLE3_WEIGHTS_I4, see below */
  int32_t append_act;    /* activations of the teacher-forced MFMA passes, see below */
  int32_t token_table;   /* embedding half of the chain step's QKV from a table, see below */
} eagle3_config;

/* Draft-KV precision.  EAGLE3_KV_F32 stores K/V rows in fp32.  EAGLE3_KV_BF16
   halves the KV bytes: every K/V element is computed at fp32 grade and stored
   rounded to the nearest bf16 (ties to even), and every read, a chain step's own
   new row included, sees the stored value.  At the drafter sizes in the tests the
   storage rounding alone moves draft logits by about 1-2e-2 against exact rows. */
#define EAGLE3_KV_F32 0
#define EAGLE3_KV_BF16 1

/* Activations of the teacher-forced (prefill / rebuild) MFMA passes of more than
   16 rows (the rows of one call, its boundary rows included, up to 4096 rows per
   pass), whose weights are exact in bf16.  Passes of at most 16 rows stream the
   weights through fp32 GEMVs in every mode.
   EAGLE3_APPEND_DEFAULT: EAGLE3_APPEND_F16 with bf16 weights, EAGLE3_APPEND_SPLIT
   with int4 weights.
   EAGLE3_APPEND_SPLIT feeds the fp32 taps and the normalised K/V-projection inputs
   [eN ; gN] as two bf16 terms hi + lo (two MFMA products, fp32-grade rows).
   EAGLE3_APPEND_BF16 rounds both to the nearest bf16 once (one product); at the
   drafter sizes in the tests that moves draft logits by 1-2.3e-2 against exact
   rows, as much as the parity bar allows, so it is only a speed option. */
#define EAGLE3_APPEND_DEFAULT 0
#define EAGLE3_APPEND_BF16 1
#define EAGLE3_APPEND_SPLIT 2
/* EAGLE3_APPEND_F16: one fp16 product.  The taps and [eN ; gN] are rounded to the
   nearest fp16 (11 significant bits against bf16's 8) and multiplied with fp16
   copies of W_fc and of the K/V rows of QKV scaled by 2^8 (a bf16 weight w times
   2^8 is exact in fp16 for 2^-25 <= |w| < 256), the products summed in fp32 and
   scaled back by 2^-8.  Half the MFMA work of SPLIT; at the drafter sizes in the
   tests draft logits stay within about 3e-3 of exact rows.  Needs bf16 weights
   (EAGLE3_E_INVAL otherwise); a tap or input outside the fp16 range, or a weight
   the scaled copy does not hold exactly, raises EAGLE3_STATUS_APPEND_RANGE (see
   eagle3_status).  0.3 GB of weight copies at the 5120-wide drafter. */
#define EAGLE3_APPEND_F16 3
/* The embedding half of a chain step's QKV projection depends on the token alone:
   W_qkv[:, :n] . RMSNorm(E[tok]) = (W_qkv[:, :n] . (input_layernorm * E[tok])) /
   rms(E[tok]) (memra_engine `eagle.rs`, module doc "Op-sequence": the embedding is
   normalised, concatenated first, then projected).  EAGLE3_TABLE_ON computes that
   value for every target token at load into an fp32 table of target_vocab x
   (n_head + 2 n_head_kv) head_dim values, and each batch-1 chain step reads one
   table row instead of streaming the embedding half of W_qkv (half of its QKV weight
   bytes).  The table is built by an MFMA GEMM whose activations,
   input_layernorm * E[tok] / rms(E[tok]) in fp32, enter as bf16 (hi, lo) pairs
   (about 2^-17 relative), summed in fp32;
   with int4 weights it multiplies the weights' exact values (scale * q, as a bf16
   hi + lo pair: two GEMMs).  EAGLE3_TABLE_DEFAULT and EAGLE3_TABLE_ON build it;
   EAGLE3_TABLE_OFF streams both halves.  3.7 GB at the Qwen3-8B shape (151936 tokens
   x 6144 rows).  Batched chains and the teacher-forced appends do not use it. */
#define EAGLE3_TABLE_DEFAULT 0
#define EAGLE3_TABLE_OFF 1
#define EAGLE3_TABLE_ON 2

/* EAGLE3_KV_Q8Q5: K rows in q8_0 and V rows in q5_1, blocks of 32 values along
   head_dim (memra_engine `eagle.rs`, `Eagle3Scratch` doc and `attn`: the draft
   layer appends quantized K/V rows and decode attention reads the quantized views;
   34 and 24 bytes per block by default).  The formulas are our reading: q8_0
   D = fp16(max|x| / 127), q = clamp(rint(x / D), -127, 127), value D q; q5_1
   D = fp16((max - min) / 31), M = fp16(min), q = clamp(rint((x - M) / D), 0, 31),
   value D q + M; every decision in fp32 on the fp32 row.  Rows are quantized once,
   when appended (teacher-forced rows as they are stored, a chain step's row by the
   attention block that owns it), and every read sees the quantized values, the new
   row's included.  Batch-1 drafting only (max_seqs 1); prefill activations keep the
   fp32-grade path of EAGLE3_KV_F32.  The quantized regions hold max_ctx + 1 rows
   rounded up to a multiple of 16 and are zeroed by eagle3_load. */
#define EAGLE3_KV_Q8Q5 2

/* Projection-weight format (ExecuTorch PR #20154 names a weight-stationary INT4
   GEMM for small M; the format is our reading).  EAGLE3_WEIGHTS_I4: eagle3_load
   quantizes fc, q/k/v, o, gate/up, down and lm_head to symmetric int4 in groups of
   32 along the input dimension with one bf16 scale per group (scale =
   bf16(max|w| / 7), q = clamp(rint(w / scale), -7, 7), IEEE fp32 divisions) and
   every draft step and append streams those (about 4.5 bits a weight).  Requires
   max_seqs == 1 and input widths (n_embd, n_head * head_dim, n_ff) that are
   multiples of 32.  Appends of at most 16 rows stream the int4 codes through the
   GEMVs; longer appends run each MFMA product twice, on the exact bf16 (hi, lo)
   halves of the int4 weights of fc and of the K/V rows. */
#define EAGLE3_WEIGHTS_BF16 0
#define EAGLE3_WEIGHTS_I4 1

/* Weights: device pointers, bf16, PyTorch [out, in] row-major (in contiguous).
   They are copied (and repacked) at load; the caller may free them afterwards.
     fc [n, 3n]; input_layernorm, hidden_norm, post_attention_layernorm, norm [n];
     q_proj [n_head*hd, 2n]; k_proj, v_proj [n_head_kv*hd, 2n]; o_proj [n, n_head*hd];
     gate_proj, up_proj [n_ff, n]; down_proj [n, n_ff]; lm_head [draft_vocab, n];
     embed [target_vocab, n] — the token embedding indexed by TARGET id (required:
     a head without an embedding table is rejected, ExecuTorch PR #20153).
   d2t_host: host int64 [draft_vocab]; target_id = draft_id + d2t[draft_id]
   (memra `d2t_map`); every target id must lie in [0, target_vocab). */
typedef struct {
  const void *fc, *input_layernorm, *hidden_norm, *q_proj, *k_proj, *v_proj, *o_proj,
      *post_attention_layernorm, *gate_proj, *up_proj, *down_proj, *norm, *lm_head, *embed;
  const int64_t *d2t_host;
  int64_t d2t_len;
  /* declared [rows, cols] of the 14 tensors above, in field order (norms: [n, 1]);
     each must equal the shape the config implies, else EAGLE3_E_SHAPE */
  int64_t shape[14][2];
} eagle3_weights;

/* Optional per-step outputs of a chain round (NULL fields are skipped):
     logits: dev fp32 [n_seq, gamma, draft_vocab] — draft logits of step j;
     hidden: dev fp32 [n_seq, gamma + 1, n_embd] — index 0 is the encoded
             boundary feature fc(aux), index j the g_next of step j. */
typedef struct {
  float *logits;
  float *hidden;
} eagle3_debug;

/* Rotary width (memra `EagleConfig::rope_dim_count` and its rope-width tests):
   an explicit rotated-dims count (rotary_dim >= 0; pass -1 if absent) wins over
   a fractional partial_factor (pass a negative value if absent), which wins over
   the full head width; a malformed factor (not in (0, 1]) takes the full width.
   An explicit count that is odd, zero or above head_dim, or a factor that does
   not give an even whole number of dims, is EAGLE3_E_UNSUPPORTED.
   Pure host function; needs no device. */
int eagle3_resolve_rope_dim(int32_t rotary_dim, float partial_factor, int32_t head_dim,
                            int32_t *out);

/* Validate the geometry (memra `Eagle3Draft::load` shape checks: fc in = 3n,
   q_proj in = 2n, q_proj out = n_head*hd, lm_head out = draft_vocab, d2t length =
   draft_vocab) and the d2t range, copy and repack the weights into library-owned
   device memory, and allocate the draft KV for max_seqs x (max_ctx + 1) rows.
   The KV is zero-initialised; every sequence starts with 0 committed rows.
   On error *out is left NULL and nothing is allocated. */
int eagle3_load(const eagle3_config *cfg, const eagle3_weights *w, void *stream,
                eagle3_ctx **out);

/* Release a handle (synchronises its device work first). NULL is a no-op. */
int eagle3_free(eagle3_ctx *ctx);

/* Teacher-forced prefill (pegainfer PR #707 `prefill_prompt`): append T rows at
   positions committed .. committed+T-1 of sequence `seq`.  Row t pairs the
   taps of target position p_t (aux*_dev[t], fp32 [T, n] each, ascending tap
   order) with tok_dev[t] (int32 [T]) = the target token at p_t + 1 (the shifted
   pairing of ExecuTorch PR #20153).  Only K and V of the rows are computed.
   Next boundary (the page's prefill also builds the boundary target feature):
   with next_aux*_dev given (fp32 [n] each: the taps of the last prompt position,
   all three or none), fc of those taps is computed in the same pass over W_fc
   and stored as the sequence's boundary feature, which a following
   eagle3_draft_chain with EAGLE3_STORED_BOUNDARY starts from; without them any
   stored feature of the sequence is dropped.
   Requires spec == 0 and committed + T <= max_ctx.  T == 0 without next taps is
   a no-op; T == 0 with them only stores the boundary feature. */
int eagle3_prefill(eagle3_ctx *ctx, int32_t seq, int32_t T, const int32_t *tok_dev,
                   const float *aux0_dev, const float *aux1_dev, const float *aux2_dev,
                   const float *next_aux0_dev, const float *next_aux1_dev,
                   const float *next_aux2_dev, void *stream);

/* One chain round per listed sequence (pegainfer PR #707 `chain_round`):
   g = fc(boundary taps), then gamma_eff greedy draft steps over the persistent
   draft KV, then rewind (unless flags & EAGLE3_KEEP_SPEC).
     seq_ids_host[n_seq]: distinct sequence slots;
     boundary_tok_dev[n_seq] (int32): the token at the boundary position;
     aux*_dev [n_seq, n] fp32: taps of the position before it; NULL with
       flags & EAGLE3_STORED_BOUNDARY, where g is each sequence's stored boundary
       feature instead (EAGLE3_E_STATE if a sequence holds none);
     out_ids_dev [n_seq, gamma] int32: target id of draft j+1, -1 beyond gamma_eff;
     gamma_eff_host[n_seq]: filled before any device work is queued,
       gamma_eff = clamp(max_ctx - committed, 0, gamma) (reserve for the k+1 commit);
     dbg: optional per-step outputs, NULL in timed runs.
   No logits leave the device; argmax and d2t run on the device. */
int eagle3_draft_chain(eagle3_ctx *ctx, int32_t n_seq, const int32_t *seq_ids_host,
                       const int32_t *boundary_tok_dev, const float *aux0_dev,
                       const float *aux1_dev, const float *aux2_dev, int32_t gamma,
                       uint32_t flags, int32_t *out_ids_dev, int32_t *gamma_eff_host,
                       const eagle3_debug *dbg, void *stream);

/* Commit accepted drafts after verification (pegainfer PR #707
   `rebuild_after_verify`): for each listed sequence b, a_b = n_accepted_host[b]
   and a_b + 1 rows are appended: (boundary taps, boundary token),
   (taps before d_1, d_1) ... (taps before d_a, d_a).  Rows are packed over
   sequences in list order: tok_dev [sum(a_b+1)] int32, aux*_dev [sum(a_b+1), n].
   Next boundary (the page's rebuild also sets the boundary target feature for
   the next round): with next_aux*_dev given ([n_seq, n] fp32 each, list order:
   the taps of each sequence's new boundary position; all three or none), their
   fc rows ride along in the same pass over W_fc and are stored as the
   sequences' boundary features for a following chain with
   EAGLE3_STORED_BOUNDARY; without them the stored features are dropped.
   Requires spec == 0, a preceding chain round on the sequence since its last
   commit, and a_b <= that round's gamma_eff. */
int eagle3_rebuild_after_verify(eagle3_ctx *ctx, int32_t n_seq, const int32_t *seq_ids_host,
                                const int32_t *n_accepted_host, const int32_t *tok_dev,
                                const float *aux0_dev, const float *aux1_dev,
                                const float *aux2_dev, const float *next_aux0_dev,
                                const float *next_aux1_dev, const float *next_aux2_dev,
                                void *stream);

/* Drop speculative rows and truncate the committed rows to new_len
   (abort / cleanup); the sequence's stored boundary feature is dropped too.
   Requires 0 <= new_len <= committed.  Host bookkeeping only: no device work.
   (pegainfer PR #707, PR description: a chain round rewinds the speculative KV so
   it has no side effects; memra_engine `eagle.rs`, `Eagle3Scratch`: the draft
   cache length is reset rather than its rows cleared.) */
int eagle3_rewind(eagle3_ctx *ctx, int32_t seq, int32_t new_len);

/* Device-side input problems since the last call (a bit mask; the call
   synchronises the device, returns the bits and clears them).  Token ids and
   logits live in device memory, so they are checked where they are used:
     EAGLE3_STATUS_BAD_TOKEN: a boundary token or a teacher-forced token outside
       [0, target_vocab) (the embedding row read is the nearest valid one);
     EAGLE3_STATUS_NAN_LOGITS: a draft step whose logits were all NaN (its draft
       id is 0, target id d2t[0]).
   A chain or append that raised a bit has produced values the caller should not
   trust. */
#define EAGLE3_STATUS_BAD_TOKEN 1u
#define EAGLE3_STATUS_NAN_LOGITS 2u
/*   EAGLE3_STATUS_APPEND_RANGE: with EAGLE3_APPEND_F16, a teacher-forced tap or
       projection input outside the fp16 range (or NaN), or (raised at load) a
       weight of W_fc or of the K/V rows that its 2^8-scaled fp16 copy does not
       hold exactly. */
#define EAGLE3_STATUS_APPEND_RANGE 4u
int eagle3_status(eagle3_ctx *ctx, uint32_t *flags);

/* Lengths of a sequence: committed rows and live speculative rows (the two
   lengths the capacity rule of pegainfer PR #707, review, "start=97, k=3,
   max=100", is stated in).  Host bookkeeping; no device work. */
int eagle3_kv_len(const eagle3_ctx *ctx, int32_t seq, int32_t *committed, int32_t *spec);

/* Copy draft-KV rows [row0, row0 + nrows) of a sequence into caller buffers
   (dev [nrows, n_head_kv, head_dim] each in the cache's element type, fp32 or
   bf16 per kv_dtype, and fp32 dequantized values for EAGLE3_KV_Q8Q5; K rows
   roped).  Inspection and tests; rows need not be live. */
int eagle3_kv_read(const eagle3_ctx *ctx, int32_t seq, int32_t row0, int32_t nrows,
                   void *k_dev, void *v_dev, void *stream);

/* Verify-window attention (the target-verify side of a round: ExecuTorch PR #20344
   "split-K mid-M SDPA ... for EAGLE-3 target_verify at long context"; PR #20156:
   one target forward per round over the K-token window).  M query rows per head,
   q_dev [M][n_head][head_dim] fp32 (roped); k_dev, v_dev [n_head_kv][cap][head_dim]
   in kv_dtype EAGLE3_KV_F32 or EAGLE3_KV_BF16 (K roped), whose rows ctx_rows ..
   ctx_rows + M - 1 hold the window's own K/V; query row m attends rows
   0 .. ctx_rows + m (scale 1/sqrt(head_dim), query head h reads KV head
   h / (n_head / n_head_kv)); out_dev [M][n_head][head_dim] fp32.  The context is
   split across blocks and the splits combined; workspace_dev must hold
   eagle3_verify_attention_workspace(...) bytes (device memory owned by the caller;
   0 bytes needed when the context fits one split).  All pointers are device
   pointers; stream is a hipStream_t (NULL: the default stream); the call is
   asynchronous.  Errors: EAGLE3_E_INVAL (null pointers, M < 1, ctx_rows < 0,
   ctx_rows + M > cap, too small a workspace), EAGLE3_E_SHAPE (n_head not a multiple
   of n_head_kv), EAGLE3_E_UNSUPPORTED (head_dim not 64/128/256, other kv_dtype). */
size_t eagle3_verify_attention_workspace(int32_t M, int32_t n_head, int32_t n_head_kv,
                                         int32_t head_dim, int32_t ctx_rows, int32_t kv_dtype);
int eagle3_verify_attention(const float *q_dev, const void *k_dev, const void *v_dev,
                            int32_t kv_dtype, int32_t cap, int32_t ctx_rows, int32_t M,
                            int32_t n_head, int32_t n_head_kv, int32_t head_dim, float *out_dev,
                            void *workspace_dev, size_t workspace_bytes, void *stream);

/* eagle3_verify_attention without a workspace argument, for callers that cannot
   allocate device memory (code under HIP graph capture, tight serving loops,
   harnesses that forbid allocation).  Same arguments, layouts, result and errors
   as eagle3_verify_attention; the split partials go to a device array inside the
   library of EAGLE3_VERIFY_SCRATCH_BYTES, of which every GPU holds one copy for the
   life of the process.  The call allocates nothing: it looks the array's address up
   on its first call on a device and launches the same kernels.  A call whose
   partials (eagle3_verify_attention_workspace bytes) exceed the array returns
   EAGLE3_E_CAPACITY before any device work; eagle3_last_error(NULL) gives the
   message of a failing call.  Calls that overlap on one GPU (e.g. on two streams)
   share the array and race; calls on one stream are ordered and safe. */
#define EAGLE3_VERIFY_SCRATCH_BYTES (16u << 20)
int eagle3_verify_attention_noalloc(const float *q_dev, const void *k_dev, const void *v_dev,
                                    int32_t kv_dtype, int32_t cap, int32_t ctx_rows, int32_t M,
                                    int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                                    float *out_dev, void *stream);

/* Copy one int4 projection matrix (weight_format EAGLE3_WEIGHTS_I4) into caller
   buffers: codes_dev [rows][K / 2] bytes and scales_dev [rows][K / 32] bf16, in the
   layout of EAGLE3_WEIGHTS_I4.  Row order as stored: fc, o_proj, down_proj and
   lm_head as given; QKV is q rows then k rows then v rows, with the q and k rows of
   each head ordered so that rotary partners are adjacent; gate/up interleaves
   gate row i (row 2i) and up row i (row 2i + 1).  Inspection and tests;
   EAGLE3_E_STATE when the weights are bf16. */
enum {
  EAGLE3_I4_FC = 0,
  EAGLE3_I4_QKV = 1,
  EAGLE3_I4_O = 2,
  EAGLE3_I4_GATE_UP = 3,
  EAGLE3_I4_DOWN = 4,
  EAGLE3_I4_LM_HEAD = 5
};
int eagle3_weights_i4_read(const eagle3_ctx *ctx, int32_t matrix, void *codes_dev,
                           void *scales_dev, void *stream);

/* Message of the last failing call on this handle (or, with ctx NULL, of the
   last failing eagle3_load or eagle3_verify_attention_noalloc on this thread).
   The library's own error reporting (no passage of the pages defines it; it
   answers pegainfer PR #707, review, which asks for clean failure paths).  The
   string stays valid until the next failing call on the same handle (with NULL:
   on the same thread) or until the handle is freed. */
const char *eagle3_last_error(const eagle3_ctx *ctx);

/* Timing of one kernel family with HIP events on the launching stream, for
   measurement.  kernel: 0 = lm_head+argmax, 1 = gate/up+SwiGLU, 2 = fused QKV (or,
   with the deferred QKV, the first step's hidden half), 3 = down, 4 = o_proj,
   5 = attention, 6 = fc encode, 7 = prefill fc GEMM, 8 = prefill K|V GEMM,
   9 = lm_head+argmax with the next step's hidden-half QKV (deferred QKV).
   enable != 0 starts a fresh accumulation. */
int eagle3_profile_enable(eagle3_ctx *ctx, int32_t kernel, int32_t enable);
/* Synchronises the recorded events and returns the summed duration and count. */
int eagle3_profile_read(eagle3_ctx *ctx, double *total_ms, int64_t *launches);

/* Calibration of the ceilings the kernels are measured against, on this GPU (no
   device memory is allocated; each result is the best of `reps` launches timed with
   HIP events on `stream`).
   eagle3_calibrate_mfma: the bf16 MFMA rate the chip sustains, in TFLOP/s: every
     wave runs four independent chains of iters v_mfma_f32_32x32x16_bf16 on
     register operands, with no memory traffic.
   eagle3_calibrate_stream: the streaming read rate of buf_dev (bytes, a multiple of
     16 is read), in GB/s, each timed read right after an untimed read of flush_dev
     (flush_bytes; larger than the 256 MB infinity cache makes buf_dev come from
     HBM).  Pointers 16-byte aligned.
   sink_dev: EAGLE3_CALIB_SINK_BYTES of device memory a never-taken branch of the
   kernels may write (it keeps their work from being optimised away). */
#define EAGLE3_CALIB_SINK_BYTES (2u << 20)
int eagle3_calibrate_mfma(int32_t iters, int32_t reps, float *sink_dev, double *tflops, void *stream);
int eagle3_calibrate_stream(const void *buf_dev, size_t bytes, const void *flush_dev, size_t flush_bytes,
                            int32_t reps, uint32_t *sink_dev, double *gbs, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE3_H */
