// The token a draft step embeds: the boundary token, or the previous step's
// draft (argmax over that step's lm_head candidates, mapped through d2t).  Used
// by the fused QKV kernels and by the attention kernels that finish a step's QKV.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

// finish the previous step (argmax over the lm_head candidates, d2t; the
// candidates' target ids come with them when prev_tok is given) or take the
// boundary token tok0; `first` is the candidates' first batch, already loaded;
// every thread of the block calls it and gets the token; the first block of
// the grid writes the outputs and status bits
template <bool MORE = true, int NT = 0>
__device__ __forceinline__ int qkv_token_from(const QkvArgs& a, const ArgmaxBatch& first, int tok0, float* sv,
                                              int* si, int* st) {
  int tok;
  if (a.prev_count > 0) {
    int bt;
    int bi = block_argmax_from<MORE, NT>(first, a.prev_val, a.prev_idx, a.prev_tok, a.prev_count, sv, si, st, &bt);
    const bool nan = bi < 0 || bi >= a.dv;  // every logit NaN
    if (nan) tok = a.d2t[0];
    else tok = a.prev_tok ? bt : bi + a.d2t[bi];
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
      *a.prev_out_id = tok;
      *a.tok_store = tok;
      if (nan) atomicOr(a.status, kStatusNanLogits);
    }
  } else {
    tok = tok0;
  }
  if (tok < 0 || tok >= a.vocab) {  // reads the nearest row, and says so
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(a.status, kStatusBadToken);
    tok = min(max(tok, 0), a.vocab - 1);
  }
  return tok;
}

// the loads qkv_token_from needs: the candidates' first batch or the boundary token
template <int NT = 0>
__device__ __forceinline__ int qkv_token_load(const QkvArgs& a, ArgmaxBatch& first) {
  if (a.prev_count > 0) {
    argmax_load<NT>(a.prev_val, a.prev_idx, a.prev_tok, a.prev_count, 0, first);
    return 0;
  }
  return *a.tok;
}

__device__ __forceinline__ int qkv_token(const QkvArgs& a, float* sv, int* si, int* st) {
  ArgmaxBatch first;
  const int tok0 = qkv_token_load(a, first);
  return qkv_token_from(a, first, tok0, sv, si, st);
}

}  // namespace e3
