// Main-kernel instantiations for head dimension 128.
#include "launch.h"

namespace detattn {
namespace {

template <int D, int BQ, int BKV, bool CAUSAL, int DQM>
MainInfo info_of() {
  static const MainInfo cached = [] {
    MainInfo m;
    auto fn = &bwd_main_kernel<D, BQ, BKV, CAUSAL, DQM>;
    m.func = reinterpret_cast<const void*>(fn);
    m.lds_bytes = MainCfg<D, BQ, BKV>::LDS_BYTES;
    m.tcopy = MainCfg<D, BQ, BKV>::TCOPY ? 1 : 0;
    int occ = 0;
    if (hipFuncSetAttribute(m.func, hipFuncAttributeMaxDynamicSharedMemorySize, m.lds_bytes) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kThreads, m.lds_bytes) != hipSuccess)
      occ = 0;
    (void)hipGetLastError();
    m.occupancy = occ;
    return m;
  }();
  return cached;
}

template <int BQ, int BKV>
MainInfo pick(int causal, int dqm) {
  if (causal) {
    if (dqm == kDqOrderedRmw) return info_of<128, BQ, BKV, true, kDqOrderedRmw>();
    if (dqm == kDqOrderedAtomic) return info_of<128, BQ, BKV, true, kDqOrderedAtomic>();
    if (dqm == kDqUnordered) return info_of<128, BQ, BKV, true, kDqUnordered>();
    if (dqm == kDqLocalRmw) return info_of<128, BQ, BKV, true, kDqLocalRmw>();
  } else {
    if (dqm == kDqOrderedRmw) return info_of<128, BQ, BKV, false, kDqOrderedRmw>();
    if (dqm == kDqOrderedAtomic) return info_of<128, BQ, BKV, false, kDqOrderedAtomic>();
    if (dqm == kDqUnordered) return info_of<128, BQ, BKV, false, kDqUnordered>();
    if (dqm == kDqLocalRmw) return info_of<128, BQ, BKV, false, kDqLocalRmw>();
  }
  return MainInfo{nullptr, 0, 0, 0};
}

}  // namespace

MainInfo main_info_d128(int BQ, int BKV, int causal, int dq_mode) {
#define X(bq, bkv) \
  if (BQ == bq && BKV == bkv) return pick<bq, bkv>(causal, dq_mode);
  X(64, 128) X(64, 64)
#undef X
  return MainInfo{nullptr, 0, 0, 0};
}

}  // namespace detattn
