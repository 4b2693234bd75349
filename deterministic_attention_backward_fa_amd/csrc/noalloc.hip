// attn_bwd_deterministic_noalloc: the deterministic backward for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation). Its workspace is this file's
// fixed device array `scratch`, one copy per GPU, held until the process ends.
#include "detattn.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = (size_t)DETATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The scratch array. In host code its name is a host-side stand-in, not a
// device address: every host use goes through the address that
// hipGetSymbolAddress returns for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr on failure.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

namespace detattn {
// The no-alloc scratch of the current device if a call has set it up there
// (detattn_device_status(NULL, ...) reads its status word), else nullptr.
void* noalloc_scratch_if_ready() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_ptr[dev];
}
}  // namespace detattn

extern "C" int attn_bwd_deterministic_noalloc(const void* q, const void* k, const void* v, const void* o,
                                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                              detattn_shape_t shape, detattn_mask_t mask,
                                              detattn_schedule_t schedule, void* stream) {
  // sizes first: a request beyond the fixed scratch is refused before any HIP call
  const size_t need = detattn_bwd_workspace_bytes(shape, mask, schedule);
  if (need == 0 && !(shape.B == 0 || shape.H == 0 || shape.S == 0)) return DETATTN_ERR_INVALID_ARG;
  if (need > kScratchBytes) return DETATTN_ERR_SCRATCH_LIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DETATTN_ERR_HIP;
  void* ws = scratch_ptr(dev);
  if (!ws) return DETATTN_ERR_HIP;
  return attn_bwd_deterministic(q, k, v, o, dout, lse, dq, dk, dv, ws, kScratchBytes, shape, mask, schedule, stream);
}
