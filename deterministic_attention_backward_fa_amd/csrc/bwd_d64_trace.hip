// Main-kernel instantiations for head dimension 64, with the per-tile phase trace.
#include "bwd_instances.h"

namespace detattn {

MainInfo main_info_d64_trace(int BQ, int BKV, int causal, int dq_mode) {
#define X(bq, bkv) \
  if (BQ == bq && BKV == bkv) return pick<64, true, bq, bkv>(causal, dq_mode);
  X(64, 64) X(128, 128) X(64, 128)
#undef X
  return MainInfo{nullptr, 0, 0};
}

}  // namespace detattn
