// Main-kernel instantiation table, included by one translation unit per head
// dimension and trace variant (the TUs compile in parallel).
#pragma once
#include "launch.h"

namespace detattn {
namespace {

template <int D, int BQ, int BKV, bool CAUSAL, int DQM, bool TRACE, bool PAIR = false>
MainInfo info_of() {
  static const MainInfo cached = [] {
    MainInfo m;
    auto fn = &bwd_main_kernel<D, BQ, BKV, CAUSAL, DQM, TRACE, PAIR>;
    m.func = reinterpret_cast<const void*>(fn);
    m.lds_bytes = MainCfg<D, BQ, BKV>::LDS_BYTES;
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

template <int D, bool TRACE, int BQ, int BKV, bool CAUSAL>
MainInfo pick_mode(int dqm) {
  switch (dqm) {
    case kDqOrderedRmw: return info_of<D, BQ, BKV, CAUSAL, kDqOrderedRmw, TRACE>();
    case kDqOrderedAtomic: return info_of<D, BQ, BKV, CAUSAL, kDqOrderedAtomic, TRACE>();
    case kDqUnordered: return info_of<D, BQ, BKV, CAUSAL, kDqUnordered, TRACE>();
    case kDqLocalRmw: return info_of<D, BQ, BKV, CAUSAL, kDqLocalRmw, TRACE>();
    case kDqUnorderedLocal: return info_of<D, BQ, BKV, CAUSAL, kDqUnorderedLocal, TRACE>();
    default: return MainInfo{nullptr, 0, 0};
  }
}

template <int D, bool TRACE, int BQ, int BKV>
MainInfo pick(int causal, int dqm) {
  return causal ? pick_mode<D, TRACE, BQ, BKV, true>(dqm) : pick_mode<D, TRACE, BQ, BKV, false>(dqm);
}

// The resident-pair instances (symmetric shift, causal; ordered dQ modes only).
template <int D, int BQ, int BKV>
MainInfo pick_pair(int dqm) {
  switch (dqm) {
    case kDqOrderedRmw: return info_of<D, BQ, BKV, true, kDqOrderedRmw, false, true>();
    case kDqOrderedAtomic: return info_of<D, BQ, BKV, true, kDqOrderedAtomic, false, true>();
    case kDqLocalRmw: return info_of<D, BQ, BKV, true, kDqLocalRmw, false, true>();
    default: return MainInfo{nullptr, 0, 0};
  }
}

}  // namespace
}  // namespace detattn
