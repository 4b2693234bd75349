// Flag hand-off latency between two workgroups, on one XCD or across XCDs: the
// MI355X counterpart of the remote-L2 hand-off the DASH pages discuss (a dQ
// tile's serialized reduction passes a flag from one SM to the next; nachedeu.com
// news piece, the inter-SM latency paragraph; zskr.cn explainer section 4.2).
//
// Workgroups wa and wb (thread 0 of each; every other workgroup exits) pass a
// counter back and forth through one 32-bit word with the same device-scope
// (agent) atomics the main kernel uses for its dQ flags: A stores 2k+1 and
// waits for 2k+2, B waits for 2k+1 and stores 2k+2, `round_trips` times. A
// records the elapsed s_memrealtime ticks (100 MHz) and s_memtime shader
// cycles; both record the XCD the hardware reports. Every wait is bounded: on
// a timeout the partner is released (the word is set to a terminal value) and
// the result records it, so the kernel always ends.
#include "detattn.h"

#include <hip/hip_runtime.h>

#include <cstring>

namespace {

constexpr unsigned kQuit = 0xFFFFFFFFu;

__device__ __forceinline__ unsigned long long rt_now() { return __builtin_amdgcn_s_memrealtime(); }

// out[0] = realtime ticks, out[1] = shader cycles, out[2] = XCD of A, out[3] = XCD of B, out[4] = 1 on timeout
__global__ __launch_bounds__(64) void xcd_pingpong_kernel(unsigned* word, int wa, int wb, int round_trips,
                                                          long long timeout_ticks, unsigned long long* out) {
  const int wg = blockIdx.x;
  if ((wg != wa && wg != wb) || threadIdx.x != 0) return;
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  out[wg == wa ? 2 : 3] = xcc & 0xF;
  const bool is_a = wg == wa;
  const unsigned long long t_start = rt_now();
  bool failed = false;
  unsigned long long r0 = 0, c0 = 0;
  for (int k = 0; k < round_trips && !failed; ++k) {
    if (is_a) {
      if (k == 1) {  // the first round trip also waits for B to start: time from the second on
        r0 = rt_now();
        c0 = __builtin_amdgcn_s_memtime();
      }
      __hip_atomic_store(word, 2u * k + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const unsigned want = is_a ? 2u * k + 2u : 2u * k + 1u;
    for (;;) {
      const unsigned v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v == want) break;
      if (v == kQuit || (long long)(rt_now() - t_start) > timeout_ticks) {
        failed = true;
        break;
      }
    }
    if (!failed && !is_a) __hip_atomic_store(word, 2u * k + 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (failed) {
    __hip_atomic_store(word, kQuit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    out[4] = 1;
  }
  if (is_a && !failed) {
    out[0] = rt_now() - r0;
    out[1] = __builtin_amdgcn_s_memtime() - c0;
  }
}

}  // namespace

extern "C" int detattn_xcd_handoff(int wg_a, int wg_b, int round_trips, void* scratch, uint64_t* result,
                                   void* stream) {
  if (wg_a < 0 || wg_b < 0 || wg_a == wg_b || wg_a >= 64 || wg_b >= 64 || round_trips < 2 || round_trips > 65536 ||
      !scratch || !result || (reinterpret_cast<uintptr_t>(scratch) & 255u) != 0 ||
      (reinterpret_cast<uintptr_t>(result) & 7u) != 0)
    return DETATTN_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned* word = static_cast<unsigned*>(scratch);
  unsigned long long* out = reinterpret_cast<unsigned long long*>(result);
  if (hipMemsetAsync(word, 0, 256, st) != hipSuccess || hipMemsetAsync(out, 0, 5 * sizeof(uint64_t), st) != hipSuccess)
    return DETATTN_ERR_HIP;
  const int grid = (wg_a > wg_b ? wg_a : wg_b) + 1;
  long long timeout = 100000000LL;  // 1 s of s_memrealtime ticks
  int a = wg_a, b = wg_b, n = round_trips;
  void* args[] = {&word, &a, &b, &n, &timeout, &out};
  // co-resident by construction: a cooperative launch fails rather than leave
  // one partner waiting for a workgroup that never starts
  const hipError_t e =
      hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&xcd_pingpong_kernel), dim3(grid), dim3(64), args, 0, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return DETATTN_ERR_HIP;
  }
  return DETATTN_OK;
}
