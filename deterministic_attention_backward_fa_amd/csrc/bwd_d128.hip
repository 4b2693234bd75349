// Main-kernel instantiations for head dimension 128, without the phase trace.
#include "bwd_instances.h"

namespace detattn {

MainInfo main_info_d128(int BQ, int BKV, int causal, int dq_mode) {
#define X(bq, bkv) \
  if (BQ == bq && BKV == bkv) return pick<128, false, bq, bkv>(causal, dq_mode);
  X(64, 128) X(64, 64)
#undef X
  return MainInfo{nullptr, 0, 0};
}

}  // namespace detattn
