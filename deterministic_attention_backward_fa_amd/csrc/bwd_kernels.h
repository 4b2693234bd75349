// Attention backward kernels for gfx950: preprocess, main (KV-stationary,
// ordered dQ accumulation), dQ convert.
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

enum DqMode : int { kDqOrderedRmw = 1, kDqOrderedAtomic = 2, kDqUnordered = 3 };

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* delta;
  float* dqacc;
  __bf16* dk;
  __bf16* dv;
  int* flags;          // one int per (head, Q tile), stride kFlagInts
  unsigned* ticket;    // dynamic item counter
  unsigned* err;       // device error word
  int BH, S;
  float scale;
  Sched sc;
  int ticket_mode;     // 1: items claimed through the ticket counter in (head, item) order
  int ring, rings;     // static rings: workgroups per ring, rings in flight
  int xcd_remap;       // place each ring on one XCD (workgroup w runs on XCD w % 8)
  long long timeout_ticks;  // s_memrealtime ticks (100 MHz)
  unsigned delay_seed;
  int skip_item;       // testing: global item index whose first signal is withheld, or -1
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

// ---------------------------------------------------------------------------
// Preprocess: D_i = sum_d dO[i,d] * O[i,d] (fp32, fixed order), zero the flags,
// the ticket and the error word, and (unordered mode) the dQ accumulator.
// 16 threads per row, each summing 8 contiguous products in order, then a
// fixed butterfly across the 16 lanes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                      float* __restrict__ delta, long long rows, int* flags,
                                                      long long n_flags, unsigned* header, float* dqacc,
                                                      long long dqacc_n4) {
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
  if (row < rows && part == 0) delta[row] = acc;
  for (long long f = gtid; f < n_flags; f += gsz) flags[f * kFlagInts] = 0;
  if (gtid < 64) header[gtid] = 0;
  if (dqacc) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (long long x = gtid; x < dqacc_n4; x += gsz) reinterpret_cast<f32x4*>(dqacc)[x] = z;
  }
}

// ---------------------------------------------------------------------------
// Main kernel
// ---------------------------------------------------------------------------
template <int D, int BQ, int BKV>
struct BwdCfg {
  static constexpr int NKVW = BKV / 32;   // waves along KV
  static constexpr int NQW = 4 / NKVW;    // waves along Q
  static constexpr int QW = BQ / NQW;     // Q rows per wave
  static constexpr int MQ = QW / 32;      // 32-row blocks of S per wave
  static constexpr int KD = D / 16;       // MFMA K steps over D
  static constexpr int ND = D / 32;       // 32-column blocks over D
  static constexpr int KQ = QW / 16;      // MFMA K steps over the wave's Q rows
  static constexpr int KKV = BKV / 16;    // MFMA K steps over the KV tile
  // dQ tile BQ x D split over the 4 waves: wave w takes D-block w % ND and
  // MQD consecutive 32-row blocks.
  static constexpr int WPD = 4 / ND;
  static constexpr int MQD = (BQ / 32) / WPD;
  static constexpr int PQ = D + 8;        // LDS pitch (elements) of Q/dO/K/V tiles
  static constexpr int PS = BQ + 8;       // LDS pitch of the transposed dS tile
  static constexpr int SQ_OFF = 0;
  static constexpr int SDO_OFF = SQ_OFF + BQ * PQ * 2;
  static constexpr int SDS_OFF = SDO_OFF + BQ * PQ * 2;
  static constexpr int SK_OFF = SDS_OFF + BKV * PS * 2;
  static constexpr int SV_OFF = SK_OFF + BKV * PQ * 2;
  static constexpr int SL_OFF = SV_OFF + BKV * PQ * 2;
  static constexpr int SD_OFF = SL_OFF + BQ * 4;
  static constexpr int TILE_BYTES = SD_OFF + BQ * 4;
  // Epilogue scratch (aliases the tile buffers): cross-wave fp32 partials
  // (NQW == 2) and the bf16 tile used for coalesced dK/dV stores.
  static constexpr int RED_BYTES = (NQW == 2) ? NKVW * 2 * ND * 16 * 64 * 4 : 0;
  static constexpr int OUT_BYTES = BKV * PQ * 2;
  static constexpr int EPI_BYTES = RED_BYTES + OUT_BYTES;
  // item broadcast slot, outside both
  static constexpr int MISC_OFF = TILE_BYTES > EPI_BYTES ? TILE_BYTES : EPI_BYTES;
  static constexpr int LDS_BYTES = MISC_OFF + 16;
  static_assert(NKVW * NQW == 4, "4 waves");
  static_assert(QW % 32 == 0 && MQD >= 1, "tile shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int D, int BQ, int BKV>
__device__ __forceinline__ void stage_rows(__bf16* dst, const __bf16* __restrict__ src, int rows) {
  using C = BwdCfg<D, BQ, BKV>;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int n = rows * CPR;
  for (int c = threadIdx.x; c < n; c += kThreads) {
    const int r = c / CPR, x = c % CPR;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + (long long)r * D + x * 8);
    lds_store16(dst + r * C::PQ + x * 8, v);
  }
}

template <int D, int BQ, int BKV, bool CAUSAL, int DQM>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using C = BwdCfg<D, BQ, BKV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __bf16* sQ = reinterpret_cast<__bf16*>(smem + C::SQ_OFF);
  __bf16* sdO = reinterpret_cast<__bf16*>(smem + C::SDO_OFF);
  __bf16* sdS = reinterpret_cast<__bf16*>(smem + C::SDS_OFF);
  __bf16* sK = reinterpret_cast<__bf16*>(smem + C::SK_OFF);
  __bf16* sV = reinterpret_cast<__bf16*>(smem + C::SV_OFF);
  float* sL = reinterpret_cast<float*>(smem + C::SL_OFF);
  float* sDl = reinterpret_cast<float*>(smem + C::SD_OFF);
  int* sMisc = reinterpret_cast<int*>(smem + C::MISC_OFF);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int wk = w % C::NKVW;
  const int wq = w / C::NKVW;
  const int nbq = w % C::ND;               // dQ: this wave's D block
  const int mq0 = (w / C::ND) * C::MQD;    // dQ: first 32-row block
  const float c1 = a.scale * kLog2e;
  const Sched sc = a.sc;
  const int ipH = sc.items_per_head();
  const long long total_items = (long long)a.BH * ipH;

  // Static ring placement.
  int ring_id = 0, slot = 0;
  if (!a.ticket_mode) {
    const int wg = blockIdx.x;
    if (a.xcd_remap) {
      const int x = wg & 7, u = wg >> 3;
      ring_id = (u / a.ring) * 8 + x;
      slot = u % a.ring;
    } else {
      ring_id = wg / a.ring;
      slot = wg % a.ring;
    }
    if (ring_id >= a.rings) return;
  }

  for (long long round = 0;; ++round) {
    // ---- claim an item ----
    long long gidx;
    if (a.ticket_mode) {
      if (tid == 0) sMisc[0] = (int)atomicAdd(a.ticket, 1u);
      __syncthreads();
      gidx = sMisc[0];
      if (gidx >= total_items) return;
    } else {
      const long long bh = (long long)ring_id + round * a.rings;
      if (bh >= a.BH) return;
      gidx = bh * ipH + slot;
    }
    const int bh = (int)(gidx / ipH);
    const int it = (int)(gidx % ipH);
    const int len = sc.item_len(it);
    const long long head_off = (long long)bh * a.S * D;

    int cur_j = -1;
    bf16x8 kB[C::KD], vB[C::KD], kTB[C::KKV];
    f32x16 dKacc[C::ND], dVacc[C::ND];

    for (int t = 0; t < len; ++t) {
      int i, j;
      sc.tile(it, t, i, j);
      if (j != cur_j) {
        // ---- new KV tile: (flush the previous one), stage K_j, V_j, fill registers ----
        cur_j = j;
        __syncthreads();
        stage_rows<D, BQ, BKV>(sK, a.k + head_off + (long long)j * BKV * D, BKV);
        stage_rows<D, BQ, BKV>(sV, a.v + head_off + (long long)j * BKV * D, BKV);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < C::KD; ++s) {
          kB[s] = frag_row(sK, C::PQ, 32 * wk, 16 * s);
          vB[s] = frag_row(sV, C::PQ, 32 * wk, 16 * s);
        }
#pragma unroll
        for (int s = 0; s < C::KKV; ++s) kTB[s] = frag_tr(sK, C::PQ, 16 * s, 32 * nbq, false);
#pragma unroll
        for (int n = 0; n < C::ND; ++n) {
          dKacc[n] = f32x16{};
          dVacc[n] = f32x16{};
        }
      }

      // ---- stage Q_i, dO_i, LSE_i (log2 units), D_i ----
      __syncthreads();
      const long long qrow0 = (long long)i * BQ;
      stage_rows<D, BQ, BKV>(sQ, a.q + head_off + qrow0 * D, BQ);
      stage_rows<D, BQ, BKV>(sdO, a.dout + head_off + qrow0 * D, BQ);
      if (tid < BQ) {
        sL[tid] = a.lse[(long long)bh * a.S + qrow0 + tid] * kLog2e;
        sDl[tid] = a.delta[(long long)bh * a.S + qrow0 + tid];
      }
      __syncthreads();

      // ---- S = Q K^T and dP = dO V^T for this wave's (QW x 32) block ----
      f32x16 sAcc[C::MQ], pAcc[C::MQ];
#pragma unroll
      for (int mb = 0; mb < C::MQ; ++mb) {
        sAcc[mb] = f32x16{};
        pAcc[mb] = f32x16{};
      }
#pragma unroll
      for (int s = 0; s < C::KD; ++s) {
#pragma unroll
        for (int mb = 0; mb < C::MQ; ++mb) {
          const bf16x8 aq = frag_row(sQ, C::PQ, C::QW * wq + 32 * mb, 16 * s);
          sAcc[mb] = mfma32(aq, kB[s], sAcc[mb]);
          const bf16x8 ad = frag_row(sdO, C::PQ, C::QW * wq + 32 * mb, 16 * s);
          pAcc[mb] = mfma32(ad, vB[s], pAcc[mb]);
        }
      }

      // ---- P and dS (elementwise, C layout: row q, column kv = lane) ----
      const bool diag = CAUSAL && ((long long)(j + 1) * BKV - 1 > qrow0);
      const int kv_glob = j * BKV + 32 * wk + c32;
      bf16x8 pB[C::KQ], dsB[C::KQ];
#pragma unroll
      for (int mb = 0; mb < C::MQ; ++mb) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int qloc = C::QW * wq + 32 * mb + 8 * rq + 4 * g;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(sL + qloc);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(sDl + qloc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e;
            float p = __builtin_amdgcn_exp2f(sAcc[mb][r] * c1 - L4[e]);
            if (diag && kv_glob > (int)qrow0 + qloc + e) p = 0.f;
            const float ds = p * (pAcc[mb][r] - D4[e]);
            const int kstep = 2 * mb + (rq >> 1);
            const int slotx = 4 * (rq & 1) + e;
            pB[kstep][slotx] = (__bf16)p;
            dsB[kstep][slotx] = (__bf16)ds;
          }
        }
      }

      // ---- dV += P^T dO, dK += dS^T Q ----
#pragma unroll
      for (int s = 0; s < C::KQ; ++s) {
#pragma unroll
        for (int n = 0; n < C::ND; ++n) {
          const bf16x8 bo = frag_tr(sdO, C::PQ, C::QW * wq + 16 * s, 32 * n, true);
          dVacc[n] = mfma32(pB[s], bo, dVacc[n]);
          const bf16x8 bq = frag_tr(sQ, C::PQ, C::QW * wq + 16 * s, 32 * n, true);
          dKacc[n] = mfma32(dsB[s], bq, dKacc[n]);
        }
      }

      // ---- dS^T -> LDS (row kv, column q), 4 consecutive q per store ----
#pragma unroll
      for (int s = 0; s < C::KQ; ++s) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = C::QW * wq + 16 * s + 8 * hh + 4 * g;
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = dsB[s][4 * hh + e];
          *reinterpret_cast<bf16x4*>(sdS + (32 * wk + c32) * C::PS + q0) = v4;
        }
      }
      __syncthreads();

      // ---- dQ partial = dS K (this wave's D block, MQD row blocks) ----
      f32x16 dqAcc[C::MQD];
#pragma unroll
      for (int m = 0; m < C::MQD; ++m) dqAcc[m] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KKV; ++s) {
#pragma unroll
        for (int m = 0; m < C::MQD; ++m) {
          const bf16x8 ad = frag_tr(sdS, C::PS, 16 * s, 32 * (mq0 + m), false);
          dqAcc[m] = mfma32(ad, kTB[s], dqAcc[m]);
        }
      }

      // ---- add into the fp32 accumulator of dQ tile i ----
      float* dqt = a.dqacc + head_off + qrow0 * D + 32 * nbq + c32;
      if constexpr (DQM == kDqUnordered) {
#pragma unroll
        for (int m = 0; m < C::MQD; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
            atomicAdd(dqt + (long long)qloc * D, dqAcc[m][r]);
          }
      } else {
        // Ordered hand-off. The accumulator is only touched through agent-scope
        // (coherent across XCDs) relaxed atomic accesses: sc1 loads/stores or fp32
        // atomic adds. Ordering: the predecessor waits until its own accesses have
        // completed (vmcnt 0 in every wave), then publishes rank+1 on the flag; the
        // successor sees the flag through an sc1 load before issuing its accesses.
        // No L2-wide writeback or invalidate is needed because no plain (possibly
        // cached, non-coherent) access to the accumulator is ever made.
        const int rk = sc.rank(i, j);
        int* flag = a.flags + ((long long)bh * sc.n_q + i) * kFlagInts;
        if (tid == 0) {
          if (a.delay_seed) {
            const long long until = now_ticks() + (hash3(a.delay_seed, (unsigned)gidx, (unsigned)t) & 1023u);
            while (now_ticks() < until) __builtin_amdgcn_s_sleep(2);
          }
          if (rk > 0) {
            const long long t0 = now_ticks();
            int spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != rk) {
              __builtin_amdgcn_s_sleep(1);
              if (((++spins) & 255) == 0) {
                if (now_ticks() - t0 > a.timeout_ticks ||
                    __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                  __hip_atomic_store(a.err, (unsigned)kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  break;
                }
              }
            }
          }
        }
        __syncthreads();
        if (rk == 0) {
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              __hip_atomic_store(dqt + (long long)qloc * D, dqAcc[m][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else if constexpr (DQM == kDqOrderedAtomic) {
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              __hip_atomic_fetch_add(dqt + (long long)qloc * D, dqAcc[m][r], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
          float old[C::MQD][16];
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              old[m][r] = __hip_atomic_load(dqt + (long long)qloc * D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              __hip_atomic_store(dqt + (long long)qloc * D, old[m][r] + dqAcc[m][r], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // every wave: its accumulator accesses are complete before the barrier
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) {
          const bool withhold = (a.skip_item >= 0 && gidx == a.skip_item && t == 0);
          if (!withhold) __hip_atomic_store(flag, rk + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }

      // ---- end of a column: epilogue (dK, dV of KV tile j to global) ----
      int ni = -1, nj = -1;
      if (t + 1 < len) sc.tile(it, t + 1, ni, nj);
      if (nj != j) {
        __syncthreads();  // every wave is done with the tile buffers
        float* red = reinterpret_cast<float*>(smem);
        __bf16* sOut = reinterpret_cast<__bf16*>(smem + C::RED_BYTES);
        if constexpr (C::NQW == 2) {
          // waves with wq == 1 hand their partial sums to the wq == 0 wave of the same KV rows
          if (wq == 1) {
#pragma unroll
            for (int n = 0; n < C::ND; ++n)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                red[(((wk * 2 + 0) * C::ND + n) * 16 + r) * 64 + lane] = dKacc[n][r];
                red[(((wk * 2 + 1) * C::ND + n) * 16 + r) * 64 + lane] = dVacc[n][r];
              }
          }
          __syncthreads();
          if (wq == 0) {
#pragma unroll
            for (int n = 0; n < C::ND; ++n)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                dKacc[n][r] = dKacc[n][r] + red[(((wk * 2 + 0) * C::ND + n) * 16 + r) * 64 + lane];
                dVacc[n][r] = dVacc[n][r] + red[(((wk * 2 + 1) * C::ND + n) * 16 + r) * 64 + lane];
              }
          }
        }
        // dK (scaled) then dV through an LDS tile for coalesced 16-byte stores
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          if (wq == 0) {
#pragma unroll
            for (int n = 0; n < C::ND; ++n)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int kv = 32 * wk + 8 * (r >> 2) + 4 * g + (r & 3);
                const float x = which == 0 ? dKacc[n][r] * a.scale : dVacc[n][r];
                sOut[kv * C::PQ + 32 * n + c32] = (__bf16)x;
              }
          }
          __syncthreads();
          __bf16* dst = (which == 0 ? a.dk : a.dv) + head_off + (long long)j * BKV * D;
          constexpr int CPR = D / 8;
          for (int cidx = tid; cidx < BKV * CPR; cidx += kThreads) {
            const int r = cidx / CPR, x = cidx % CPR;
            *reinterpret_cast<bf16x8*>(dst + (long long)r * D + x * 8) = lds_load16(sOut + r * C::PQ + x * 8);
          }
          __syncthreads();
        }
      }
    }
  }
}

}  // namespace detattn
