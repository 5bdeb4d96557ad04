/*
 * eagle3_trunk.h — the verify side of a speculative round on the GPU: a small
 * Llama-style target trunk and a greedy speculative-decoding runner that drives it
 * together with the drafter of eagle3.h.
 *
 * One round follows the runner semantics of ExecuTorch PR #20156 ("Add the EAGLE-3
 * speculative-decoding runner (CUDA)", description: one target forward over the
 * K-token window per round; greedy verification keeps the output identical to
 * plain greedy decoding) and PR #20153 ("Add the Eagle3Speculator module",
 * description: target_verify returns the per-position argmax; the next chain is
 * reseeded from the features the verify forward produced, the target feature of
 * position t paired with token t + 1).  The accept walk, the bonus token and the
 * cache rollback are those of memra_engine `eagle.rs`, `generate_spec_eagle`.
 *
 * The trunk stands in for a target model at test width: every output of a row is
 * computed in a fixed order that does not depend on the window it is part of, so
 * the runner's tokens equal greedy decoding of the same trunk one token at a time.
 *
 * Conventions are those of eagle3.h (int status codes, "dev" = device pointer,
 * streams as void*, checks before any device work, one host thread per handle).
 */
#ifndef EAGLE3_TRUNK_H
#define EAGLE3_TRUNK_H

#include <stdint.h>

#include "eagle3.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct eagle3_trunk eagle3_trunk;

typedef struct {
  int32_t n_embd, n_head, n_head_kv, head_dim;  /* head_dim 64, 128 or 256 */
  int32_t n_ff, vocab, n_layers;                /* n_layers >= 2 */
  float rope_theta, rms_eps;                    /* full-width NeoX rotary embedding */
  int32_t max_ctx;                              /* rows of the trunk KV cache */
  int32_t max_tokens;                           /* largest window of one forward */
} eagle3_trunk_config;

/* Device pointers, bf16, PyTorch [out, in] row-major, copied at load:
     embed [vocab, n] (token embedding), final_norm [n], lm_head [vocab, n] (untied);
     layers: n_layers * 9 pointers, layer by layer: attn_norm [n], wq [n_head*hd, n],
     wk [n_head_kv*hd, n], wv [n_head_kv*hd, n], wo [n, n_head*hd], mlp_norm [n],
     w_gate [n_ff, n], w_up [n_ff, n], w_down [n, n_ff];
   shapes: (3 + 9 * n_layers) declared [rows, cols] pairs in the same order (embed,
   final_norm, lm_head, then the layers; norms [n, 1]), each checked against the
   config (EAGLE3_E_SHAPE). */
typedef struct {
  const void *embed, *final_norm, *lm_head;
  const void *const *layers;
  const int64_t *shapes;
} eagle3_trunk_weights;

/* Validate, copy the weights, allocate the KV cache (n_layers x 2 x n_head_kv x
   max_ctx x head_dim fp32) and scratch for windows of max_tokens rows.  On error
   *out stays NULL and nothing stays allocated. */
int eagle3_trunk_load(const eagle3_trunk_config *cfg, const eagle3_trunk_weights *w, void *stream,
                      eagle3_trunk **out);
int eagle3_trunk_free(eagle3_trunk *t);

/* One forward over T tokens (tok_dev int32 [T]) at positions len .. len + T - 1
   (the verify window, a prompt, or one decode step): appends T rows to the cache
   and writes ids_dev [T] = the greedy token after each position (argmax of the
   logits, lowest index on ties) and, for each non-NULL tap pointer, fp32 [T, n]:
   tap0 = the residual stream entering layer 0 (the embedding), tap1 = leaving layer
   n_layers / 2 - 1, tap2 = leaving the last layer (before the final norm).  Query
   row t attends over cache rows 0 .. len + t.  Requires 1 <= T <= max_tokens and
   len + T <= max_ctx (EAGLE3_E_CAPACITY).  An input id outside [0, vocab) is read
   as id 0 and raises EAGLE3_TRUNK_BAD_TOKEN in the status word. */
int eagle3_trunk_forward(eagle3_trunk *t, int32_t T, const int32_t *tok_dev, int32_t *ids_dev,
                         float *tap0_dev, float *tap1_dev, float *tap2_dev, void *stream);

/* Truncate the cache to new_len rows (0 <= new_len <= len); host bookkeeping. */
int eagle3_trunk_rollback(eagle3_trunk *t, int32_t new_len);
int eagle3_trunk_len(const eagle3_trunk *t, int32_t *len);

/* Status bits raised by the trunk's kernels since the last call; synchronises the
   trunk's last stream and clears the word. */
#define EAGLE3_TRUNK_BAD_TOKEN 1u   /* an input id outside the vocabulary */
#define EAGLE3_TRUNK_NAN_LOGITS 2u  /* a position whose logits were all NaN */
int eagle3_trunk_status(eagle3_trunk *t, uint32_t *flags);

const char *eagle3_trunk_last_error(const eagle3_trunk *t);

/* Greedy speculative decoding on the device.  The trunk is reset (len 0) and the
   drafter's sequence `seq` rewound to 0, then:
     prompt: one trunk forward over the prompt gives its taps and x_P (the greedy
       token after it, emitted first); the drafter is prefilled with the rows
       (taps of r, x_{r+1}), r < prompt_len - 1, and stores the boundary feature of
       the taps of position prompt_len - 1;
     each round: eagle3_draft_chain from the stored boundary (gamma_eff drafts);
       one trunk forward over [x_n, d_1 .. d_gamma_eff] (the verify window); the
       accept walk on the device gives a (the longest prefix with d_{i+1} equal to
       the trunk's token after position n + i) and the bonus token; d_1 .. d_a and
       the bonus are emitted (up to max_new tokens in all); the trunk rolls back to
       n + a + 1 rows; eagle3_rebuild_after_verify commits (taps of n - 1, x_n),
       (taps of n, d_1) .. (taps of n + a - 1, d_a) and stores the boundary feature
       of the taps of position n + a; the bonus is the next boundary token.
   One device-to-host copy of (a, bonus, drafts) per round is the only
   synchronisation.  out_host receives max_new tokens; drafted / accepted (host,
   may be NULL) the totals.  Requires matching widths (trunk n_embd == drafter
   n_embd, trunk vocab == drafter target_vocab, else EAGLE3_E_SHAPE), 1 <= prompt_len
   <= max_tokens, gamma + 1 <= max_tokens, prompt_len + max_new + gamma <= the
   trunk's max_ctx, and a drafter whose max_ctx admits prompt_len + max_new rows
   (EAGLE3_E_CAPACITY); any drafter or trunk error ends the call with that code. */
int eagle3_generate(eagle3_ctx *drafter, int32_t seq, eagle3_trunk *trunk, const int32_t *prompt_host,
                    int32_t prompt_len, int32_t max_new, int32_t gamma, int32_t *out_host,
                    int64_t *drafted, int64_t *accepted, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE3_TRUNK_H */
