// Attention backward for gfx950: launch arguments, the preprocess kernel, and
// (bwd_main.h) the main KV-stationary kernel with ordered dQ accumulation.
//
// Main kernel design. A persistent workgroup of 4 waves owns one item at a
// time: a KV tile j (BKV rows) whose K_j, V_j live in registers and whose
// dK_j, dV_j fp32 accumulators stay in registers across the whole Q-tile sweep
// (all work of a KV tile stays on one compute unit: DASH, zskr.cn explainer
// 2.2; gist.science summary 2.1). Wave w covers KV rows 32*(w % NKVW) ..+31
// and Q rows QW*(w / NKVW) ..+QW-1 of each Q tile. Per visited Q tile i:
//   S  = Q_i K_j^T,  dP = dO_i V_j^T            (bf16 MFMA, fp32 acc)
//   P  = exp(scale*S - LSE_i) [0 where masked], dS = P (dP - D_i)
//   dV_j += P^T dO_i,  dK_j += dS^T Q_i           (P, dS rounded to bf16)
//   dQ_i partial = dS K_j                         (dS transposed via LDS)
// and the partial is added to the fp32 dQ accumulator of tile i after every
// earlier contributor in that tile's fixed order has added its own: a flag per
// dQ tile counts the adds done (FA3's serialized reduction, explainer 2.1;
// summary 1). dQ = scale * accumulator is rounded to bf16 by the convert
// kernel; dK is scaled in the epilogue.
#pragma once
#include "common.h"
#include "tile_sched.h"

namespace detattn {

// kDqLocalRmw: ordered read-modify-write whose accumulator and flag accesses
// use sc0 (L2-coherent) instead of sc1 (coherent across XCDs); valid only when
// every workgroup touching a head's dQ tiles runs on one XCD.
enum DqMode : int {
  kDqOrderedRmw = 1,       // ordered read-modify-write, device scope
  kDqOrderedAtomic = 2,    // ordered fp32 atomic adds, device scope
  kDqUnordered = 3,        // unordered fp32 atomic adds, device scope (non-deterministic)
  kDqLocalRmw = 4,         // ordered read-modify-write in one XCD's L2
  kDqUnorderedLocal = 5    // unordered fp32 atomic adds in one XCD's L2 (non-deterministic)
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* nlse;   // -LSE / scale per row (initial value of the S accumulator)
  const float* ndelta; // -D per row (initial value of the dP accumulator)
  float* dqacc;
  __bf16* dk;
  __bf16* dv;
  int* flags;          // one int per (head, Q tile), stride kFlagInts
  unsigned* ticket;    // dynamic item counter
  unsigned* err;       // error bits of this call (workspace header, kHdrAbort)
  unsigned* sticky;    // error bits kept until the status is read (kHdrSticky)
  unsigned* xcd_tab;   // XCD registration: per workgroup, 1 + the XCD it runs on (0: not yet registered)
  int BH, S;
  float scale;
  Sched sc;
  int ticket_mode;     // 1: items claimed through the ticket counter in (head, item) order
  int ring, rings;     // static rings: workgroups per ring, rings in flight
  int snake;           // static rings: odd rounds give slot g item kG + G-1-g (rank independent)
  int xcd_remap;       // rings of one XCD: membership from the XCD each workgroup runs on
  long long timeout_ticks;  // s_memrealtime ticks (100 MHz)
  unsigned delay_seed;
  int skip_item;       // testing: global item index whose first signal is withheld, or -1
  int misplace;        // testing: XCD-local rings start from a wrong guess (workgroup w takes w+1's place)
  unsigned long long* trace;  // optional per-workgroup phase timestamps
  int trace_records;
};

static constexpr int kFlagInts = (int)(WsLayout::kFlagStride / 4);
static constexpr int kThreads = 256;

__device__ __forceinline__ unsigned hash3(unsigned a, unsigned b, unsigned c) {
  unsigned h = a * 0x9E3779B1u ^ (b + 0x7F4A7C15u) * 0x85EBCA77u ^ (c + 0x165667B1u) * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return h;
}

__device__ __forceinline__ long long now_ticks() { return (long long)__builtin_amdgcn_s_memrealtime(); }

// A device-side failure: the call's abort word (every later wait of the call
// gives up at once) and the sticky status word (read by detattn_device_status).
__device__ __forceinline__ void report_error(const BwdArgs& a, unsigned bits) {
  __hip_atomic_fetch_or(a.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_or(a.sticky, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Preprocess: D_i = sum_d dO[i,d] * O[i,d] (fp32, fixed order); the main
// kernel's accumulator initial values -D_i and -LSE_i * log2(e); zero the
// flags and the per-call header words (ticket, abort word, XCD registration),
// initialise the sticky status word on a workspace's first use, and
// (unordered mode) zero the dQ accumulator.
// 16 threads per row, each summing 8 contiguous products in order, then a
// fixed butterfly across the 16 lanes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ nlse, float* __restrict__ ndelta,
                                                      long long rows, int* flags,
                                                      long long n_flags, unsigned* header, unsigned* xcd_tab,
                                                      int n_tab, float* dqacc, long long dqacc_n4) {
  constexpr int TPR = D / 8;  // threads per row
  constexpr int RPB = 256 / TPR;
  const long long gtid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long gsz = (long long)gridDim.x * 256;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * D + part * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * D + part * 8);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += (float)a[t] * (float)b[t];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < rows && part == 0) {
    ndelta[row] = -acc;
    nlse[row] = -lse[row] * kLog2e;
  }
  for (long long f = gtid; f < n_flags; f += gsz) flags[f * kFlagInts] = 0;
  if (gtid < kHdrZeroWords) header[gtid] = 0;
  for (long long x = gtid; x < n_tab; x += gsz) xcd_tab[x] = 0;  // a workgroup's entry is its arrival
  if (gtid == 0) {
    unsigned long long* tag = reinterpret_cast<unsigned long long*>(header + kHdrTag);
    if (*tag != kStickyTag) {
      header[kHdrSticky] = 0;
      *tag = kStickyTag;
    }
  }
  if (dqacc) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (long long x = gtid; x < dqacc_n4; x += gsz) reinterpret_cast<f32x4*>(dqacc)[x] = z;
  }
}

// ---------------------------------------------------------------------------

}  // namespace detattn

#include "bwd_main.h"
