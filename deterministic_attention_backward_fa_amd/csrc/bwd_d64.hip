// Main-kernel instantiations for head dimension 64, without the phase trace.
#include "bwd_instances.h"

namespace detattn {

MainInfo main_info_d64(int BQ, int BKV, int causal, int dq_mode) {
#define X(bq, bkv) \
  if (BQ == bq && BKV == bkv) return pick<64, false, bq, bkv>(causal, dq_mode);
  X(64, 64) X(128, 128) X(64, 128)
#undef X
  return MainInfo{nullptr, 0, 0};
}

// Resident-pair symmetric shift: both columns' K, V, K^T, dK, dV fit the 256
// AGPRs at D = 64 with 64 x 64 tiles (112 per column).
MainInfo main_info_d64_pair(int BQ, int BKV, int dq_mode) {
  if (BQ == 64 && BKV == 64) return pick_pair<64, 64, 64>(dq_mode);
  return MainInfo{nullptr, 0, 0};
}

}  // namespace detattn
