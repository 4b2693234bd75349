// Launchers of the preprocess, convert and forward kernels, and of the main
// backward kernel (plain or cooperative grid).
#include "fwd_kernels.h"
#include "launch.h"

namespace detattn {

// dQ = bf16_rne(scale * acc), 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                          long long n8, float scale) {
  const long long gsz = (long long)gridDim.x * 256;
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n8; x += gsz) {
    const f32x4 a = reinterpret_cast<const f32x4*>(acc)[2 * x];
    const f32x4 b = reinterpret_cast<const f32x4*>(acc)[2 * x + 1];
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      r[t] = (__bf16)(scale * a[t]);
      r[4 + t] = (__bf16)(scale * b[t]);
    }
    reinterpret_cast<bf16x8*>(dq)[x] = r;
  }
}


static int grid_for(long long work_items, int per_block, int cap) {
  long long g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

hipError_t launch_pre(int D, const __bf16* o, const __bf16* dout, const float* lse, float inv_scale, float* nlse,
                      float* ndelta,
                      long long rows, int* flags,
                      long long n_flags, unsigned* header, float* dqacc, long long dqacc_elems, hipStream_t st) {
  const int rpb = 256 / (D / 8);
  long long g = (rows + rpb - 1) / rpb;
  if (g < 1) g = 1;
  // the same grid also zeroes the flags and (unordered mode) the accumulator with grid-stride loops
  const long long dq4 = dqacc ? dqacc_elems / 4 : 0;
  if (D == 64)
    bwd_pre_kernel<64><<<dim3((unsigned)g), dim3(256), 0, st>>>(o, dout, lse, inv_scale, nlse, ndelta, rows, flags, n_flags, header, dqacc, dq4);
  else
    bwd_pre_kernel<128><<<dim3((unsigned)g), dim3(256), 0, st>>>(o, dout, lse, inv_scale, nlse, ndelta, rows, flags, n_flags, header,
                                                                 dqacc, dq4);
  return hipGetLastError();
}

hipError_t launch_transpose(int D, const __bf16* q, const __bf16* dout, __bf16* qt, __bf16* dot, long long BH, int S,
                            hipStream_t st) {
  const dim3 grid((unsigned)(S / 64), (unsigned)BH);
  if (D == 64)
    bwd_transpose_kernel<64><<<grid, dim3(256), 0, st>>>(q, dout, qt, dot, S);
  else
    bwd_transpose_kernel<128><<<grid, dim3(256), 0, st>>>(q, dout, qt, dot, S);
  return hipGetLastError();
}

hipError_t launch_convert(const float* acc, __bf16* dq, long long elems, float scale, hipStream_t st) {
  const long long n8 = elems / 8;
  const int g = grid_for(n8, 256, 256 * 16);
  bwd_convert_kernel<<<dim3(g), dim3(256), 0, st>>>(acc, dq, n8, scale);
  return hipGetLastError();
}

hipError_t launch_main(const MainLaunch& L, hipStream_t st) {
  MainInfo info = L.D == 64 ? main_info_d64(L.BQ, L.BKV, L.causal, L.dq_mode)
                            : main_info_d128(L.BQ, L.BKV, L.causal, L.dq_mode);
  if (!info.func) return hipErrorInvalidDeviceFunction;
  BwdArgs args = L.args;
  void* kargs[] = {(void*)&args};
  if (L.cooperative)
    return hipLaunchCooperativeKernel(info.func, dim3(L.grid), dim3(kThreads), kargs, (unsigned)info.lds_bytes, st);
  return hipLaunchKernel(info.func, dim3(L.grid), dim3(kThreads), kargs, (size_t)info.lds_bytes, st);
}

hipError_t launch_fwd(int D, int causal, const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse,
                      int BH, int S, float scale, hipStream_t st) {
  dim3 grid((unsigned)(S / FwdCfg<64>::BQ), (unsigned)BH);
  if (D == 64) {
    if (causal) fwd_kernel<64, true><<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
    else fwd_kernel<64, false><<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
  } else {
    if (causal) fwd_kernel<128, true><<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
    else fwd_kernel<128, false><<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
  }
  return hipGetLastError();
}

}  // namespace detattn
