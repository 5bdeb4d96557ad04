/*
 * eagle3_ledger.h — the draft-KV length bookkeeping used inside the eagle3
 * engine, exported on its own so host code (and the CPU test-suite) can drive
 * exactly the rules the engine applies, without a device.
 *
 * Rules (pegainfer PR #707 review of the capacity check: a fully accepted
 * chain of k drafts commits k + 1 rows; reserve that row or shrink k):
 *   rows held per sequence = max_ctx + 1;
 *   prefill of T rows: spec == 0 and committed + T <= max_ctx;
 *   chain: spec == 0, 0 <= gamma <= max_gamma,
 *          gamma_eff = clamp(max_ctx - committed, 0, gamma);
 *          spec := gamma_eff with EAGLE3_KEEP_SPEC, else 0 (rewound);
 *   rebuild of a accepted drafts: spec == 0, a chain since the last commit,
 *          0 <= a <= its gamma_eff, committed + a + 1 <= max_ctx + 1;
 *          committed += a + 1;
 *   rewind to new_len: 0 <= new_len <= committed; spec := 0.
 * Boundary feature: prefill / rebuild with_boundary != 0 leave a stored
 *   boundary feature, without it they drop it, rewind drops it; a chain with
 *   flags & EAGLE3_STORED_BOUNDARY needs one (else EAGLE3_E_STATE).  A prefill
 *   of T == 0 without a boundary changes nothing.
 * Round-local chain (flags & EAGLE3_ROUND_LOCAL): spec == 0 and the gamma range
 *   as above; gamma_eff = gamma; nothing changes (EAGLE3_KEEP_SPEC with it is
 *   EAGLE3_E_INVAL).
 * Every call returns EAGLE3_OK or an EAGLE3_E_* code and changes nothing on
 * error.  Host memory only.
 */
#ifndef EAGLE3_LEDGER_H
#define EAGLE3_LEDGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct eagle3_ledger eagle3_ledger;

int eagle3_ledger_create(int32_t max_ctx, int32_t max_seqs, int32_t max_gamma,
                         eagle3_ledger **out);
void eagle3_ledger_destroy(eagle3_ledger *l);
int eagle3_ledger_prefill(eagle3_ledger *l, int32_t seq, int32_t T, int32_t with_boundary);
int eagle3_ledger_chain(eagle3_ledger *l, int32_t seq, int32_t gamma, uint32_t flags,
                        int32_t *gamma_eff);
int eagle3_ledger_rebuild(eagle3_ledger *l, int32_t seq, int32_t n_accepted,
                          int32_t with_boundary);
int eagle3_ledger_rewind(eagle3_ledger *l, int32_t seq, int32_t new_len);
int eagle3_ledger_len(const eagle3_ledger *l, int32_t seq, int32_t *committed, int32_t *spec);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE3_LEDGER_H */
