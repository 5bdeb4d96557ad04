// Launch configurations of the GEMV family: (id, waves per block, rows per
// wave, 16-byte chunk steps in flight per lane).  Rows per wave must be even
// for the kernels whose epilogue pairs rows (fused QKV, gate/up).
#pragma once

#define E3_GEMV_CONFIGS(X) \
  X(0, 4, 4, 2)            \
  X(1, 8, 2, 4)            \
  X(2, 8, 1, 8)            \
  X(3, 4, 2, 4)            \
  X(4, 8, 4, 2)            \
  X(5, 4, 1, 8)            \
  X(6, 8, 2, 8)            \
  X(7, 16, 1, 8)           \
  X(8, 4, 2, 8)            \
  X(9, 16, 2, 4)           \
  X(10, 8, 2, 2)           \
  X(11, 8, 2, 6)           \
  X(12, 16, 2, 2)          \
  X(13, 16, 2, 6)

namespace e3 {

constexpr int kGemvConfigCount = 14;

// rows per wave of a configuration (-1: no such configuration)
inline int gemv_cfg_rows(int cfg) {
  switch (cfg) {
#define E3_CFG_ROWS(ID, WV, RR, UU) \
  case ID:                          \
    return RR;
    E3_GEMV_CONFIGS(E3_CFG_ROWS)
#undef E3_CFG_ROWS
    default:
      return -1;
  }
}

enum GemvKind { kGemvEncode = 0, kGemvQkv, kGemvO, kGemvGateUp, kGemvDown, kGemvLmHead, kGemvKinds };

// tuned choice per kind (rows/K of the drafter shapes).  int4 rows are a quarter
// of the bytes, so those kernels keep a whole row (K / 32 chunks: two chunk steps
// for K = 4096, six for K = 12288) in flight per lane.
inline int gemv_pick(int kind, int N, int K, bool i4 = false) {
  (void)N;
  if (i4) {
    const int steps = (K / 32 + 63) / 64;
    switch (kind) {
      case kGemvQkv: return 10;  // two halves per row set: R = 2 keeps it in 128 VGPRs
      case kGemvGateUp: return 10;
      case kGemvLmHead: return 10;
      default: return steps > 2 ? 11 : 10;
    }
  }
  switch (kind) {
    case kGemvEncode: return 1;
    case kGemvQkv: return 8;
    case kGemvO: return 1;
    case kGemvGateUp: return 1;
    case kGemvDown: return 1;
    case kGemvLmHead: return 1;
    default: return 0;
  }
}

}  // namespace e3
