// Launchers of the preprocess, convert and forward kernels, and of the main
// backward kernel (plain or cooperative grid).
#include "fwd_kernels.h"

#include <cfloat>

#include "launch.h"

namespace detattn {

// dQ = bf16_rne(scale * acc) from a row-major accumulator, 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_convert_rm_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
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

// dQ = bf16_rne(scale * acc) from an accumulator in fragment order
// (described in common.h): a workgroup takes 32-row blocks, reads each block's 16-byte
// runs, and writes the rows through LDS as 16-byte runs.
template <int D>
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                          long long row_blocks, float scale) {
  constexpr int PITCH = D + 8;          // bf16 per LDS row (16-byte aligned rows)
  constexpr int RUNS_IN = D / 32 * 256;  // 16-byte accumulator runs per row block
  __shared__ __attribute__((aligned(16))) __bf16 tile[32 * PITCH];
  for (long long rb = blockIdx.x; rb < row_blocks; rb += gridDim.x) {
    const f32x4* src = reinterpret_cast<const f32x4*>(acc + rb * 32 * D);
    for (int c = threadIdx.x; c < RUNS_IN; c += 256) {
      const f32x4 v = src[c];
      // run c: column block c / 256, register group h, lane (g, column c % 32)
      const int h = (c >> 6) & 3, ln = c & 63;
      const int row = 8 * h + 4 * (ln >> 5), col = (c >> 8) * 32 + (ln & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[(row + e) * PITCH + col] = (__bf16)(scale * v[e]);
    }
    __syncthreads();
    for (int x = threadIdx.x; x < 32 * D / 8; x += 256) {
      const int row = x / (D / 8), c8 = x % (D / 8);
      reinterpret_cast<bf16x8*>(dq + (rb * 32 + row) * D)[c8] = *reinterpret_cast<const bf16x8*>(tile + row * PITCH + c8 * 8);
    }
    __syncthreads();
  }
}

static int grid_for(long long work_items, int per_block, int cap) {
  long long g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

hipError_t launch_pre(int D, const __bf16* o, const __bf16* dout, const float* lse, float* nlse,
                      float* ndelta,
                      long long rows, int* flags,
                      long long n_flags, unsigned* header, unsigned* xcd_tab, int n_tab, float* dqacc,
                      long long dqacc_elems, hipStream_t st) {
  const int rpb = 256 / (D / 8);
  long long g = (rows + rpb - 1) / rpb;
  if (g < 1) g = 1;
  // the same grid also zeroes the flags and (unordered mode) the accumulator with grid-stride loops
  const long long dq4 = dqacc ? dqacc_elems / 4 : 0;
  if (D == 64)
    bwd_pre_kernel<64><<<dim3((unsigned)g), dim3(256), 0, st>>>(o, dout, lse, nlse, ndelta, rows, flags, n_flags, header,
                                                                xcd_tab, n_tab, dqacc, dq4);
  else
    bwd_pre_kernel<128><<<dim3((unsigned)g), dim3(256), 0, st>>>(o, dout, lse, nlse, ndelta, rows, flags, n_flags, header,
                                                                 xcd_tab, n_tab, dqacc, dq4);
  return hipGetLastError();
}

hipError_t launch_convert(int D, const float* acc, __bf16* dq, long long rows, float scale, bool fragment_order,
                          hipStream_t st) {
  if (!fragment_order) {
    const long long n8 = rows * D / 8;
    const int g = grid_for(n8, 256, 256 * 16);
    bwd_convert_rm_kernel<<<dim3(g), dim3(256), 0, st>>>(acc, dq, n8, scale);
    return hipGetLastError();
  }
  const long long rb = rows / 32;
  const int g = grid_for(rb, 1, 256 * 16);
  if (D == 64)
    bwd_convert_kernel<64><<<dim3(g), dim3(256), 0, st>>>(acc, dq, rb, scale);
  else
    bwd_convert_kernel<128><<<dim3(g), dim3(256), 0, st>>>(acc, dq, rb, scale);
  return hipGetLastError();
}

hipError_t launch_main(const MainLaunch& L, hipStream_t st) {
  MainInfo info = main_info(L.D, L.BQ, L.BKV, L.causal, L.dq_mode, L.args.trace != nullptr, L.pair != 0);
  if (!info.func) return hipErrorInvalidDeviceFunction;
  BwdArgs args = L.args;
  void* kargs[] = {(void*)&args};
  if (L.cooperative)
    return hipLaunchCooperativeKernel(info.func, dim3(L.grid), dim3(kThreads), kargs, (unsigned)info.lds_bytes, st);
  return hipLaunchKernel(info.func, dim3(L.grid), dim3(kThreads), kargs, (size_t)info.lds_bytes, st);
}

hipError_t launch_fwd(int D, int causal, const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse,
                      int BH, int S, float scale, hipStream_t st) {
  dim3 grid((unsigned)BH, (unsigned)(S / FwdCfg<64>::BQ));
  // the kernel's own factor, computed the same way: the raw-score maximum
  // needs it positive and normal (any scale > 0 that does not overflow)
  const float c1 = scale * kLog2e;
  const bool raw = c1 >= FLT_MIN && c1 <= FLT_MAX;
  if (D == 64) {
    if (causal) (raw ? fwd_kernel<64, true, true> : fwd_kernel<64, true, false>)<<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
    else (raw ? fwd_kernel<64, false, true> : fwd_kernel<64, false, false>)<<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
  } else {
    if (causal) (raw ? fwd_kernel<128, true, true> : fwd_kernel<128, true, false>)<<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
    else (raw ? fwd_kernel<128, false, true> : fwd_kernel<128, false, false>)<<<grid, 256, 0, st>>>(q, k, v, o, lse, S, scale);
  }
  return hipGetLastError();
}

}  // namespace detattn
