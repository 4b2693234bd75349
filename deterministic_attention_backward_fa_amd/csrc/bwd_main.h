// Main attention-backward kernel for gfx950 (KV-stationary, ordered dQ).
//
// A persistent workgroup of 4 waves owns one item at a time: a KV tile j
// (BKV rows, or the two KV tiles of a symmetric pair one after the other)
// whose K_j, V_j live in registers and whose dK_j, dV_j fp32 accumulators stay
// in registers across the whole Q-tile sweep: all work of a KV tile stays on
// one compute unit (DASH, zskr.cn explainer 2.2; gist.science summary 2.1).
// Wave w covers KV rows 32*(w % NKVW) .. +31 and Q rows QW*(w / NKVW) ..
// +QW-1 of each Q tile. Per visited Q tile i:
//   S  = Q_i K_j^T,  dP = dO_i V_j^T             (bf16 MFMA, fp32 accumulate)
//   P  = exp(scale*S - LSE_i) [0 where masked],  dS = P (dP - D_i)
//   dQ_i partial = dS K_j                          (dS transposed through LDS)
//   dV_j += P^T dO_i,  dK_j += dS^T Q_i            (P, dS rounded to bf16)
// The dQ partial is added to the fp32 accumulator of tile i only after every
// earlier contributor in that tile's fixed order has added its own: a flag per
// dQ tile counts the adds done (the serialized reduction of FA3's
// deterministic mode, explainer 2.1, summary 1; the schedules in
// tile_sched.h decide the order). dQ = scale * accumulator is rounded to bf16
// by the convert kernel; dK is scaled in the epilogue.
//
// Pipeline per tile t (buffer b = t & 1):
//   top:  wait for this tile's LDS-DMA data and the previous tile's dQ adds,
//         barrier, publish the previous tile's flag, start the DMA of tile t+1
//         (Q, dO, LSE, D) into buffer b^1;
//   S, dP, P, dS; dS^T -> LDS; barrier; dQ partial (MFMA);
//   each wave waits (one lane polling) for the tile's flag, then issues its
//   adds (fp32 atomic adds, or sc1 stores for the first contributor);
//   dV, dK MFMAs run while those adds are in flight.
// The accumulator is touched only through agent-scope coherent accesses, so
// the hand-off needs no cache writeback or invalidate: "all adds done" is
// vmcnt 0 in every wave before the barrier that precedes the flag store.
#pragma once
#include "common.h"
#include "tile_sched.h"

#include <type_traits>

namespace detattn {

template <int D, int BQ, int BKV>
struct MainCfg {
  static constexpr int NKVW = BKV / 32;  // waves along KV
  static constexpr int NQW = 4 / NKVW;   // waves along Q
  static constexpr int QW = BQ / NQW;    // Q rows per wave
  static constexpr int MQ = QW / 32;     // 32-row blocks of S per wave
  static constexpr int KD = D / 16;      // MFMA K steps over D
  static constexpr int ND = D / 32;      // 32-column blocks over D
  static constexpr int KQ = QW / 16;     // MFMA K steps over the wave's Q rows
  static constexpr int KKV = BKV / 16;   // MFMA K steps over the KV tile
  static constexpr int WPD = 4 / ND;     // waves per D block of the dQ tile
  static constexpr int MQD = (BQ / 32) / WPD;
  static constexpr int NCH_D = D / 8;    // 16-byte chunks per Q/dO/K/V row
  static constexpr int NCH_S = BQ / 8;   // 16-byte chunks per dS^T row
  static constexpr int Q_BYTES = BQ * D * 2;
  static constexpr int K_BYTES = BKV * D * 2;
  static constexpr int S_BYTES = BKV * BQ * 2;
  static constexpr int LD_BYTES = BQ * 4 * 2;  // LSE then D
  static constexpr int OFF_Q0 = 0;
  static constexpr int OFF_Q1 = OFF_Q0 + Q_BYTES;
  static constexpr int OFF_DO0 = OFF_Q1 + Q_BYTES;
  static constexpr int OFF_DO1 = OFF_DO0 + Q_BYTES;
  static constexpr int OFF_LD0 = OFF_DO1 + Q_BYTES;
  static constexpr int OFF_LD1 = OFF_LD0 + LD_BYTES;
  static constexpr int OFF_DS = OFF_LD1 + LD_BYTES;
  static constexpr int OFF_K = OFF_DS + S_BYTES;
  static constexpr int OFF_V = OFF_K + K_BYTES;
  static constexpr int TILE_END = OFF_V + K_BYTES;
  // Epilogue scratch, aliasing the tile buffers (nothing is in flight then):
  // per output tensor, the fp32 partials of the waves with wq == 1 (NQW == 2)
  // and a padded bf16 tile for coalesced stores.
  static constexpr int PO = D + 8;
  static constexpr int RED_BYTES = (NQW == 2) ? NKVW * 32 * D * 4 : 0;
  static constexpr int OUT_BYTES = BKV * PO * 2;
  static constexpr int EPI_END = RED_BYTES + OUT_BYTES;
  static constexpr int OFF_MISC = TILE_END > EPI_END ? TILE_END : EPI_END;
  static constexpr int LDS_BYTES = OFF_MISC + 16;
  static_assert(NKVW * NQW == 4, "4 waves");
  static_assert(QW % 32 == 0 && MQD >= 1, "tile shape");
  static_assert((BQ * D / 8) % 256 == 0 && (BKV * D / 8) % 256 == 0, "DMA granularity");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Epilogue of one KV tile: (NQW == 2) fold the wq == 1 waves' partial sums into
// the wq == 0 waves, round to bf16 (times `mul`) through a padded LDS tile and
// store BKV x D with 16-byte coalesced writes.
template <class C>
__device__ __forceinline__ void store_column(f32x16 (&acc)[C::ND], float mul, __bf16* __restrict__ dst, float* red,
                                             __bf16* sOut, int wk, int wq, int lane) {
  constexpr int D = C::ND * 32;
  constexpr int BKV = C::NKVW * 32;
  const int g = lane >> 5, c32 = lane & 31, tid = threadIdx.x;
  if constexpr (C::NQW == 2) {
    if (wq == 1) {
#pragma unroll
      for (int n = 0; n < C::ND; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wk * C::ND + n) * 16 + r) * 64 + lane] = acc[n][r];
    }
    __syncthreads();
    if (wq == 0) {
#pragma unroll
      for (int n = 0; n < C::ND; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[n][r] = acc[n][r] + red[((wk * C::ND + n) * 16 + r) * 64 + lane];
    }
  }
  if (wq == 0) {
#pragma unroll
    for (int n = 0; n < C::ND; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = 32 * wk + 8 * (r >> 2) + 4 * g + (r & 3);
        sOut[kv * C::PO + 32 * n + c32] = (__bf16)(acc[n][r] * mul);
      }
  }
  __syncthreads();
  constexpr int CPR = D / 8;
  for (int cidx = tid; cidx < BKV * CPR; cidx += kThreads) {
    const int r = cidx / CPR, x = cidx % CPR;
    *reinterpret_cast<bf16x8*>(dst + (long long)r * D + x * 8) = lds_load16(sOut + r * C::PO + x * 8);
  }
  __syncthreads();
}

template <int D, int BQ, int BKV, bool CAUSAL, int DQM>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using C = MainCfg<D, BQ, BKV>;
  // Scope of the accumulator accesses: across XCDs (sc1), or inside the XCD's
  // L2 (sc0) when every workgroup of a ring runs on one XCD. sc0 loads may hit
  // the compute unit's own L1, so that mode invalidates L1 (buffer_inv sc0)
  // after observing the flag and before loading. Flags always use sc1.
  constexpr int kScope = DQM == kDqLocalRmw ? __HIP_MEMORY_SCOPE_WORKGROUP : __HIP_MEMORY_SCOPE_AGENT;
  constexpr int kFlagScope = __HIP_MEMORY_SCOPE_AGENT;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __bf16* sK = reinterpret_cast<__bf16*>(smem + C::OFF_K);
  __bf16* sV = reinterpret_cast<__bf16*>(smem + C::OFF_V);
  __bf16* sdS = reinterpret_cast<__bf16*>(smem + C::OFF_DS);
  int* sMisc = reinterpret_cast<int*>(smem + C::OFF_MISC);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int wk = w % C::NKVW;
  const int wq = w / C::NKVW;
  const int nbq = w % C::ND;             // dQ: this wave's D block
  const int mq0 = (w / C::ND) * C::MQD;  // dQ: first 32-row block
  const float c1 = a.scale * kLog2e;
  const Sched sc = a.sc;
  const int ipH = sc.items_per_head();
  const long long total_items = (long long)a.BH * ipH;

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
    if constexpr (DQM == kDqLocalRmw) {
      // the ring placement assumes workgroup w runs on XCD w % 8: verify it
      unsigned xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      if (tid == 0 && (int)(xcc & 0xF) != (wg & 7))
        __hip_atomic_fetch_or(a.err, (unsigned)kErrPlacement, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Q, dO, LSE and D of Q tile i -> buffer b (asynchronous).
  auto dma_q = [&](int b, long long head_off, long long bhS, int i) {
    const long long qrow0 = (long long)i * BQ;
    __bf16* dq_ = reinterpret_cast<__bf16*>(smem + (b ? C::OFF_Q1 : C::OFF_Q0));
    __bf16* ddo = reinterpret_cast<__bf16*>(smem + (b ? C::OFF_DO1 : C::OFF_DO0));
    float* ld = reinterpret_cast<float*>(smem + (b ? C::OFF_LD1 : C::OFF_LD0));
    dma_tile<C::NCH_D>(dq_, a.q + head_off + qrow0 * D, BQ);
    dma_tile<C::NCH_D>(ddo, a.dout + head_off + qrow0 * D, BQ);
    dma_f32(ld, a.lse2 + bhS + qrow0, BQ, 0);
    dma_f32(ld + BQ, a.delta + bhS + qrow0, BQ, 1);
  };

  // Optional phase trace: wave 0, lane 0 of each workgroup.
  int trace_n = 0;
  auto trace_rec = [&](int phase, int t, long long item) {
    if (a.trace && tid == 0 && trace_n < a.trace_records) {
      unsigned long long* p = a.trace + ((size_t)blockIdx.x * a.trace_records + trace_n) * 2;
      p[0] = __builtin_amdgcn_s_memtime();
      p[1] = (unsigned long long)phase | ((unsigned long long)(t & 0xFFFFFF) << 8) | ((unsigned long long)item << 32);
      ++trace_n;
    }
  };

  for (long long round = 0;; ++round) {
    long long gidx;
    if (a.ticket_mode) {
      if (tid == 0) sMisc[0] = (int)atomicAdd(a.ticket, 1u);
      __syncthreads();
      gidx = sMisc[0];
      __syncthreads();
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
    const long long bhS = (long long)bh * a.S;

    int* pend_flag = nullptr;  // flag of the previous tile, published once its adds are complete
    int pend_val = 0;

    for (int seg = 0; seg < sc.segments(); ++seg) {
    const int t_begin = sc.seg_begin(it, seg), t_end = sc.seg_end(it, seg);
    int i0, j;
    sc.tile(it, t_begin, i0, j);
    // ---- segment prologue: K_j, V_j and the first Q tile, synchronously ----
    dma_tile<C::NCH_D>(sK, a.k + head_off + (long long)j * BKV * D, BKV);
    dma_tile<C::NCH_D>(sV, a.v + head_off + (long long)j * BKV * D, BKV);
    dma_q(0, head_off, bhS, i0);
    wait_vm_all();
    __syncthreads();
    bf16x8 kB[C::KD], vB[C::KD], kTB[C::KKV];
#pragma unroll
    for (int s = 0; s < C::KD; ++s) {
      kB[s] = frag_row_s<C::NCH_D>(sK, 32 * wk, 16 * s);
      vB[s] = frag_row_s<C::NCH_D>(sV, 32 * wk, 16 * s);
    }
#pragma unroll
    for (int s = 0; s < C::KKV; ++s) kTB[s] = frag_tr_s<C::NCH_D>(sK, 16 * s, 32 * nbq, false);
    f32x16 dKacc[C::ND], dVacc[C::ND];
#pragma unroll
    for (int n = 0; n < C::ND; ++n) {
      dKacc[n] = f32x16{};
      dVacc[n] = f32x16{};
    }
    trace_rec(6, t_begin, gidx);

    int t = t_begin;
    do {
      int i, jj;
      sc.tile(it, t, i, jj);
      const int b = (t - t_begin) & 1;
      const long long qrow0 = (long long)i * BQ;
      trace_rec(0, t, gidx);
      // prefetch the next tile of this column into the other buffer
      if (t + 1 < t_end) {
        int ni, nj;
        sc.tile(it, t + 1, ni, nj);
        dma_q(b ^ 1, head_off, bhS, ni);
      }
      const __bf16* sQ = reinterpret_cast<const __bf16*>(smem + (b ? C::OFF_Q1 : C::OFF_Q0));
      const __bf16* sdO = reinterpret_cast<const __bf16*>(smem + (b ? C::OFF_DO1 : C::OFF_DO0));
      const float* sL = reinterpret_cast<const float*>(smem + (b ? C::OFF_LD1 : C::OFF_LD0));
      const float* sDl = sL + BQ;

      // Per 32-row block mb of this wave's Q rows the work is: S and dP
      // (2*KD MFMAs), the elementwise P/dS (VALU), and dV/dK over the block's
      // two K steps (4*ND MFMAs). Blocks are pipelined so that the MFMAs of one
      // block run while the VALU of the previous one executes; the last
      // block's dV/dK is deferred until after the dQ hand-off, where it covers
      // the latency of the accumulator adds.
      const bool diag = CAUSAL && ((long long)(j + 1) * BKV - 1 > qrow0);
      // kv - q offset of this lane's column against the tile's first Q row;
      // pushed far below any q when the tile needs no mask (branch-free).
      const int kv_rel = diag ? (int)((long long)j * BKV - qrow0) + 32 * wk + c32 : -(1 << 30);
      f32x16 sAcc[C::MQ], pAcc[C::MQ];
      bf16x8 pB[C::KQ], dsB[C::KQ];

      // Operand fragments are software-pipelined one K step ahead: the loads
      // of step s+1 are issued before the MFMAs of step s (sched_barrier keeps
      // the compiler from regrouping them), so LDS latency overlaps the MFMAs.
      auto sdp = [&](int mb) {
        sAcc[mb] = f32x16{};
        pAcc[mb] = f32x16{};
        bf16x8 aq = frag_row_s<C::NCH_D>(sQ, C::QW * wq + 32 * mb, 0);
        bf16x8 ad = frag_row_s<C::NCH_D>(sdO, C::QW * wq + 32 * mb, 0);
#pragma unroll
        for (int s = 0; s < C::KD; ++s) {
          bf16x8 aqn = aq, adn = ad;
          if (s + 1 < C::KD) {
            aqn = frag_row_s<C::NCH_D>(sQ, C::QW * wq + 32 * mb, 16 * (s + 1));
            adn = frag_row_s<C::NCH_D>(sdO, C::QW * wq + 32 * mb, 16 * (s + 1));
          }
          __builtin_amdgcn_sched_barrier(0);
          sAcc[mb] = mfma32(aq, kB[s], sAcc[mb]);
          pAcc[mb] = mfma32(ad, vB[s], pAcc[mb]);
          __builtin_amdgcn_sched_barrier(0);
          aq = aqn;
          ad = adn;
        }
      };
      auto elem = [&](int mb) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int qloc = C::QW * wq + 32 * mb + 8 * rq + 4 * g;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(sL + qloc);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(sDl + qloc);
          float p[4], ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e;
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sAcc[mb][r], c1, -L4[e]));
            p[e] = kv_rel > qloc + e ? 0.f : p[e];
            ds[e] = p[e] * (pAcc[mb][r] - D4[e]);
          }
          const int kstep = 2 * mb + (rq >> 1);
          const int sl = 4 * (rq & 1);
          const bf16x2 p01 = cvt2(p[0], p[1]), p23 = cvt2(p[2], p[3]);
          const bf16x2 d01 = cvt2(ds[0], ds[1]), d23 = cvt2(ds[2], ds[3]);
          pB[kstep][sl] = p01[0];
          pB[kstep][sl + 1] = p01[1];
          pB[kstep][sl + 2] = p23[0];
          pB[kstep][sl + 3] = p23[1];
          dsB[kstep][sl] = d01[0];
          dsB[kstep][sl + 1] = d01[1];
          dsB[kstep][sl + 2] = d23[0];
          dsB[kstep][sl + 3] = d23[1];
        }
      };
      auto dvdk = [&](int mb) {
        bf16x8 bo = frag_tr_s<C::NCH_D>(sdO, C::QW * wq + 16 * (2 * mb), 0, true);
        bf16x8 bq = frag_tr_s<C::NCH_D>(sQ, C::QW * wq + 16 * (2 * mb), 0, true);
#pragma unroll
        for (int x = 0; x < 2 * C::ND; ++x) {
          const int s = 2 * mb + x / C::ND, n = x % C::ND;
          bf16x8 bon = bo, bqn = bq;
          if (x + 1 < 2 * C::ND) {
            const int s1 = 2 * mb + (x + 1) / C::ND, n1 = (x + 1) % C::ND;
            bon = frag_tr_s<C::NCH_D>(sdO, C::QW * wq + 16 * s1, 32 * n1, true);
            bqn = frag_tr_s<C::NCH_D>(sQ, C::QW * wq + 16 * s1, 32 * n1, true);
          }
          __builtin_amdgcn_sched_barrier(0);
          dVacc[n] = mfma32(pB[s], bo, dVacc[n]);
          dKacc[n] = mfma32(dsB[s], bq, dKacc[n]);
          __builtin_amdgcn_sched_barrier(0);
          bo = bon;
          bq = bqn;
        }
      };

      sdp(0);
#pragma unroll
      for (int mb = 1; mb < C::MQ; ++mb) {
        sdp(mb);
        elem(mb - 1);
        if (mb >= 2) dvdk(mb - 2);
      }
      elem(C::MQ - 1);
      if (C::MQ >= 2) dvdk(C::MQ - 2);

      // ---- dS^T -> LDS (row kv, column q), 4 consecutive q per 8-byte store ----
#pragma unroll
      for (int s = 0; s < C::KQ; ++s) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = C::QW * wq + 16 * s + 8 * hh + 4 * g;
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = dsB[s][4 * hh + e];
          *reinterpret_cast<bf16x4*>(sdS + swz_off<C::NCH_S>(32 * wk + c32, q0)) = v4;
        }
      }
      trace_rec(1, t, gidx);

      // The dQ tile's flag is read now; the load completes under the barrier
      // and the dQ MFMAs, and is only re-polled if the turn has not come yet.
      const int rk = DQM == kDqUnordered ? 0 : sc.rank(i, j);
      int* flag = a.flags + ((long long)bh * sc.n_q + i) * kFlagInts;
      int seen = rk;
      if (DQM != kDqUnordered && rk > 0 && lane == 0) seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, kFlagScope);
      __syncthreads();

      // ---- dQ partial = dS K (this wave's D block, MQD row blocks) ----
      f32x16 dqAcc[C::MQD];
#pragma unroll
      for (int m = 0; m < C::MQD; ++m) dqAcc[m] = f32x16{};
      {
        bf16x8 ad[C::MQD];
#pragma unroll
        for (int m = 0; m < C::MQD; ++m) ad[m] = frag_tr_s<C::NCH_S>(sdS, 0, 32 * (mq0 + m), false);
#pragma unroll
        for (int s = 0; s < C::KKV; ++s) {
          bf16x8 adn[C::MQD];
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
            adn[m] = s + 1 < C::KKV ? frag_tr_s<C::NCH_S>(sdS, 16 * (s + 1), 32 * (mq0 + m), false) : ad[m];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < C::MQD; ++m) dqAcc[m] = mfma32(ad[m], kTB[s], dqAcc[m]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < C::MQD; ++m) ad[m] = adn[m];
        }
      }
      trace_rec(2, t, gidx);

      // ---- add the partial into dQ tile i's fp32 accumulator ----
      float* dqt = a.dqacc + head_off + qrow0 * D + 32 * nbq + c32;
      if constexpr (DQM == kDqUnordered) {
        __builtin_amdgcn_sched_barrier(0);  // same scheduling region boundary as the ordered modes' turn wait
#pragma unroll
        for (int m = 0; m < C::MQD; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
            __hip_atomic_fetch_add(dqt + (long long)qloc * D, dqAcc[m][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
      } else {
        if (lane == 0) {
          if (a.delay_seed) {
            const long long until = now_ticks() + (hash3(a.delay_seed, (unsigned)gidx, (unsigned)(t * 4 + w)) & 1023u);
            while (now_ticks() < until) __builtin_amdgcn_s_sleep(2);
          }
          if (seen != rk) {
            const long long t0 = now_ticks();
            int spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, kFlagScope) != rk) {
              __builtin_amdgcn_s_sleep(1);
              if (((++spins) & 255) == 0) {
                if (now_ticks() - t0 > a.timeout_ticks ||
                    __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                  __hip_atomic_fetch_or(a.err, (unsigned)kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  break;
                }
              }
            }
          }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        trace_rec(3, t, gidx);
        if (rk == 0) {
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              __hip_atomic_store(dqt + (long long)qloc * D, dqAcc[m][r], __ATOMIC_RELAXED, kScope);
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
          if constexpr (DQM == kDqLocalRmw) asm volatile("buffer_inv sc0" ::: "memory");
          float old[C::MQD][16];
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              old[m][r] = __hip_atomic_load(dqt + (long long)qloc * D, __ATOMIC_RELAXED, kScope);
            }
#pragma unroll
          for (int m = 0; m < C::MQD; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qloc = 32 * (mq0 + m) + 8 * (r >> 2) + 4 * g + (r & 3);
              __hip_atomic_store(dqt + (long long)qloc * D, old[m][r] + dqAcc[m][r], __ATOMIC_RELAXED, kScope);
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const bool withhold = (a.skip_item >= 0 && gidx == a.skip_item && t == 0);
        pend_flag = withhold ? nullptr : flag;
        pend_val = rk + 1;
      }
      trace_rec(4, t, gidx);
      // the last block's dV/dK runs while the adds are in flight
      dvdk(C::MQ - 1);

      trace_rec(5, t, gidx);
      ++t;
      if (t >= t_end) break;
      // the next tile's DMA (issued during this tile) and this tile's
      // accumulator adds are complete in every wave
      wait_vm_all();
      __syncthreads();
      if (tid == 0 && pend_flag)
        __hip_atomic_store(pend_flag, pend_val, __ATOMIC_RELAXED, kFlagScope);
      pend_flag = nullptr;
    } while (true);  // tiles of the segment

    // ---- end of a column: publish, then dK, dV of KV tile j to global ----
    wait_vm_all();
    __syncthreads();
    if (tid == 0 && pend_flag) __hip_atomic_store(pend_flag, pend_val, __ATOMIC_RELAXED, kFlagScope);
    pend_flag = nullptr;
    {
      float* red = reinterpret_cast<float*>(smem);
      __bf16* sOut = reinterpret_cast<__bf16*>(smem + C::RED_BYTES);
      store_column<C>(dKacc, a.scale, a.dk + head_off + (long long)j * BKV * D, red, sOut, wk, wq, lane);
      store_column<C>(dVacc, 1.f, a.dv + head_off + (long long)j * BKV * D, red, sOut, wk, wq, lane);
    }
    trace_rec(7, t_end, gidx);
    }  // segments
  }  // items
}

}  // namespace detattn
