// Internal interface between the C ABI (capi.cpp) and the kernel translation
// units (one per head dimension, so their template instantiations compile in
// parallel).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_kernels.h"

namespace detattn {

struct MainLaunch {
  BwdArgs args;
  int D, BQ, BKV, causal, dq_mode;  // dq_mode: DqMode
  int pair;                          // resident-pair symmetric shift instance
  int grid;
  int cooperative;
};

// Kernel attributes for one main-kernel instantiation.
struct MainInfo {
  const void* func;  // kernel symbol, or nullptr if the combination is not built
  int lds_bytes;
  int occupancy;     // workgroups per compute unit (0 if unknown)
};

MainInfo main_info_d64(int BQ, int BKV, int causal, int dq_mode);
MainInfo main_info_d64_pair(int BQ, int BKV, int dq_mode);
MainInfo main_info_d128(int BQ, int BKV, int causal, int dq_mode);
MainInfo main_info_d64_trace(int BQ, int BKV, int causal, int dq_mode);
MainInfo main_info_d128_trace(int BQ, int BKV, int causal, int dq_mode);

// The instance for head dimension D (64 or 128); `trace` selects the variant
// that writes the per-tile phase trace, `pair` the resident-pair symmetric
// shift (built at D = 64 with 64 x 64 tiles, causal, untraced).
inline MainInfo main_info(int D, int BQ, int BKV, int causal, int dq_mode, bool trace, bool pair = false) {
  if (pair) return (D == 64 && causal && !trace) ? main_info_d64_pair(BQ, BKV, dq_mode) : MainInfo{nullptr, 0, 0};
  if (D == 64) return trace ? main_info_d64_trace(BQ, BKV, causal, dq_mode) : main_info_d64(BQ, BKV, causal, dq_mode);
  if (D == 128) return trace ? main_info_d128_trace(BQ, BKV, causal, dq_mode) : main_info_d128(BQ, BKV, causal, dq_mode);
  return MainInfo{nullptr, 0, 0};
}

hipError_t launch_pre(int D, const __bf16* o, const __bf16* dout, const float* lse, float* nlse,
                      float* ndelta,
                      long long rows, int* flags,
                      long long n_flags, unsigned* header, unsigned* xcd_tab, int n_tab, float* dqacc,
                      long long dqacc_elems, hipStream_t st);
// fragment_order: the accumulator layout of the read-modify-write dQ modes
// (described in common.h); otherwise row-major (atomic modes)
hipError_t launch_convert(int D, const float* acc, __bf16* dq, long long rows, float scale, bool fragment_order,
                          hipStream_t st);
hipError_t launch_main(const MainLaunch& L, hipStream_t st);
hipError_t launch_fwd(int D, int causal, const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse,
                      int BH, int S, float scale, hipStream_t st);

}  // namespace detattn
