// Host-side draft-KV bookkeeping: committed rows, live speculative rows and
// the gamma_eff of the last chain round per sequence.
//
// Capacity rule (pegainfer PR #707, review of the capacity check: a fully
// accepted chain of k drafts commits k + 1 rows, so either reserve the extra
// row or shrink k at the edge — both are done here):
//   rows allocated per sequence      = max_ctx + 1
//   chain admission                  gamma_eff = clamp(max_ctx - committed, 0, gamma)
//   rebuild of a accepted drafts     a <= gamma_eff of the preceding chain and
//                                    committed + a + 1 <= max_ctx + 1
//   prefill of T rows                committed + T <= max_ctx
// A chain round writes rows committed .. committed + gamma_eff - 1 and is
// rewound afterwards (its rows become dead) unless the caller keeps them.
// Boundary feature: prefill and rebuild may also encode the taps of the next
// round's boundary (the pages' prefill and rebuild_after_verify set the boundary
// target feature); the sequence then holds a stored feature until the next
// prefill, rebuild or rewind, and a chain round may start from it.
// Round-local chains (the scratch-KV drafter of memra_engine `eagle.rs`: a draft KV
// emptied every round) attend only over their own rows: gamma_eff = gamma, and no
// length, speculative count or rebuild permission changes.
#pragma once

#include <stdint.h>

#include <vector>

#include "../../include/eagle3.h"

namespace e3 {

class Ledger {
 public:
  struct Seq {
    int32_t committed = 0;
    int32_t spec = 0;
    int32_t last_gamma = -1;  // -1: no chain since the last commit
    bool boundary = false;    // a stored boundary feature for the current length
  };

  Ledger() = default;
  Ledger(int32_t max_ctx, int32_t max_seqs, int32_t max_gamma)
      : max_ctx_(max_ctx), max_gamma_(max_gamma), seqs_(size_t(max_seqs)) {}

  int32_t rows() const { return max_ctx_ + 1; }
  int32_t max_ctx() const { return max_ctx_; }
  int32_t max_gamma() const { return max_gamma_; }
  int32_t n_seqs() const { return int32_t(seqs_.size()); }
  bool valid_seq(int32_t s) const { return s >= 0 && s < n_seqs(); }
  const Seq& seq(int32_t s) const { return seqs_[size_t(s)]; }

  // ---- checks: return a status, never mutate ----
  int check_prefill(int32_t s, int32_t T, const char** why) const {
    if (!valid_seq(s)) return fail(why, "bad sequence id", EAGLE3_E_INVAL);
    if (T < 0) return fail(why, "negative row count", EAGLE3_E_INVAL);
    const Seq& q = seq(s);
    if (q.spec) return fail(why, "speculative rows are live", EAGLE3_E_STATE);
    if (int64_t(q.committed) + T > max_ctx_) return fail(why, "prefill past max_ctx", EAGLE3_E_CAPACITY);
    return EAGLE3_OK;
  }

  int admit_chain(int32_t s, int32_t gamma, bool stored_boundary, bool round_local,
                  int32_t* gamma_eff, const char** why) const {
    if (!valid_seq(s)) return fail(why, "bad sequence id", EAGLE3_E_INVAL);
    if (gamma < 0 || gamma > max_gamma_) return fail(why, "gamma out of range", EAGLE3_E_INVAL);
    const Seq& q = seq(s);
    if (q.spec) return fail(why, "speculative rows are live", EAGLE3_E_STATE);
    if (stored_boundary && !q.boundary)
      return fail(why, "no stored boundary feature for this sequence", EAGLE3_E_STATE);
    if (round_local) {
      *gamma_eff = gamma;
      return EAGLE3_OK;
    }
    int32_t room = max_ctx_ - q.committed;
    if (room < 0) room = 0;
    *gamma_eff = gamma < room ? gamma : room;
    return EAGLE3_OK;
  }

  int check_rebuild(int32_t s, int32_t a, const char** why) const {
    if (!valid_seq(s)) return fail(why, "bad sequence id", EAGLE3_E_INVAL);
    const Seq& q = seq(s);
    if (q.spec) return fail(why, "speculative rows are live", EAGLE3_E_STATE);
    if (q.last_gamma < 0) return fail(why, "rebuild without a preceding chain round", EAGLE3_E_STATE);
    if (a < 0 || a > q.last_gamma)
      return fail(why, "accepted count exceeds the chain's gamma_eff", EAGLE3_E_INVAL);
    if (int64_t(q.committed) + a + 1 > rows())
      return fail(why, "rebuild past the reserved row", EAGLE3_E_CAPACITY);
    return EAGLE3_OK;
  }

  int check_rewind(int32_t s, int32_t new_len, const char** why) const {
    if (!valid_seq(s)) return fail(why, "bad sequence id", EAGLE3_E_INVAL);
    if (new_len < 0 || new_len > seq(s).committed)
      return fail(why, "rewind target outside [0, committed]", EAGLE3_E_INVAL);
    return EAGLE3_OK;
  }

  // ---- transitions: call only after the matching check succeeded ----
  int32_t do_prefill(int32_t s, int32_t T, bool boundary) {
    Seq& q = seqs_[size_t(s)];
    const int32_t start = q.committed;
    q.committed += T;
    q.last_gamma = -1;
    q.boundary = boundary;
    return start;
  }
  void do_chain(int32_t s, int32_t gamma_eff, bool keep_spec) {
    Seq& q = seqs_[size_t(s)];
    q.spec = keep_spec ? gamma_eff : 0;
    q.last_gamma = gamma_eff;
  }
  int32_t do_rebuild(int32_t s, int32_t a, bool boundary) {
    Seq& q = seqs_[size_t(s)];
    const int32_t start = q.committed;
    q.committed += a + 1;
    q.last_gamma = -1;
    q.boundary = boundary;
    return start;
  }
  void do_rewind(int32_t s, int32_t new_len) {
    Seq& q = seqs_[size_t(s)];
    q.committed = new_len;
    q.spec = 0;
    q.last_gamma = -1;
    q.boundary = false;
  }

 private:
  static int fail(const char** why, const char* msg, int code) {
    if (why) *why = msg;
    return code;
  }
  int32_t max_ctx_ = 0, max_gamma_ = 0;
  std::vector<Seq> seqs_;
};

}  // namespace e3
