// Attention forward for gfx950: produces O (bf16) and LSE (fp32, natural log),
// the inputs of the backward. Deterministic by construction: each output row
// is owned by one wave and reduced in a fixed order.
//
// A workgroup of 4 waves owns 128 query rows (32 per wave, kept in registers)
// and streams KV tiles of 64 rows through LDS. At D = 64 the next tile's K, V
// are loaded into registers while the current one is computed (at D = 128 the
// extra registers cost more occupancy than the overlap gains; there the tile
// goes straight from global memory to LDS by LDS-DMA). The D = 128
// instances are held to 168 registers, three waves per SIMD, and the D = 64
// ones to 128, four waves (the causal instances spill a few registers there
// and are still faster than with fewer waves). Under a causal mask the query
// blocks with the most KV tiles run first, those of every head before any
// lighter block. Each wave computes the scores
// transposed, S^T = K Q^T, so that in the MFMA accumulator layout every lane
// owns one query (its column) and the running max / sum of the online softmax
// are per-lane scalars; O^T = V^T P^T then takes P^T straight from the
// accumulator registers, and the rescaling of O^T is per lane as well.
#pragma once
#include "common.h"

namespace detattn {

template <int D>
struct FwdCfg {
  static constexpr int BQ = 128;
  static constexpr int BKV = 64;
  static constexpr int KD = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int MK = BKV / 32;   // 32-row KV blocks per tile
  static constexpr int KK = BKV / 16;   // K steps over a KV tile
  static constexpr int P = D + 8;       // LDS pitch
  static constexpr int LDS_BYTES = 2 * BKV * P * 2;
  static constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  static constexpr int NPT = BKV * CPR / 256;    // chunks per thread per tile
  static_assert(NPT * 256 == BKV * CPR, "tile chunks split evenly over 256 threads");
  static constexpr bool PREFETCH = D <= 64;     // K, V of the next tile in registers
  static constexpr bool DMA = !PREFETCH;        // else K, V go through LDS-DMA
  // LDS-DMA of a tile: 16-byte chunks in padded-row order (D / 8 data chunks
  // and one padding chunk per row, P * 2 bytes), 1 KB per instruction
  static constexpr int NCH = D / 8;
  static constexpr int DMA_INS = BKV * (NCH + 1) / 64;
  static_assert(BKV * (NCH + 1) % 64 == 0 && P * 2 == (NCH + 1) * 16, "DMA tile layout");
};

// RAW_MAX (taken when scale * log2(e) is a positive normal float): the tile
// maximum is found on the raw scores and scaled once. Rounding to nearest is
// monotonic, so for a positive factor this is exactly the maximum of the
// rounded products, one multiply per tile instead of one per score; the
// exponent arguments are fma(s, c1, -m) either way.
template <int D, bool CAUSAL, bool RAW_MAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 3 : 4))) void fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                     const __bf16* __restrict__ v, __bf16* __restrict__ o,
                                                     float* __restrict__ lse, int S, float scale) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[C::BKV * C::P];
  __shared__ __attribute__((aligned(16))) __bf16 sV[C::BKV * C::P];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, c32 = lane & 31;
  // the grid is (head, query block) and workgroups are dispatched x-fastest,
  // so under a causal mask every head's heaviest query block goes first
  const int bh = blockIdx.x;
  const int qb = CAUSAL ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y;  // query block
  const int q0 = qb * C::BQ + 32 * w;  // this wave's first query row
  const long long head = (long long)bh * S * D;
  const float c1 = scale * kLog2e;

  // Q^T as B operand: lane holds Q[q0 + c32][16s + 8g .. +7]
  bf16x8 qB[C::KD];
#pragma unroll
  for (int s = 0; s < C::KD; ++s)
    qB[s] = *reinterpret_cast<const bf16x8*>(q + head + (long long)(q0 + c32) * D + 16 * s + 8 * g);

  f32x16 oAcc[C::ND];
#pragma unroll
  for (int n = 0; n < C::ND; ++n) oAcc[n] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;  // log2 units; per lane = per query q0 + c32
  const int qi = q0 + c32;

  const int kv_end = CAUSAL ? (qb + 1) * C::BQ : S;
  // thread tid moves chunks tid, tid + 256, ... of a tile: row cidx / CPR, chunk cidx % CPR
  bf16x8 kr[C::NPT], vr[C::NPT];
  auto load_tile = [&](int kv) {
#pragma unroll
    for (int x = 0; x < C::NPT; ++x) {
      const int cidx = tid + 256 * x, r = cidx / C::CPR, c = cidx % C::CPR;
      kr[x] = *reinterpret_cast<const bf16x8*>(k + head + (long long)(kv + r) * D + 8 * c);
      vr[x] = *reinterpret_cast<const bf16x8*>(v + head + (long long)(kv + r) * D + 8 * c);
    }
  };
  // LDS-DMA: instruction ins moves chunks 64 ins .. + 63 of the padded tile
  // (row p / (NCH + 1), chunk p % (NCH + 1)); a padding chunk re-reads its
  // row's first chunk, whose bytes land in the padding and are never read
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto dma_tile = [&](int kv) {
    const unsigned char* gk = reinterpret_cast<const unsigned char*>(k + head + (long long)kv * D);
    const unsigned char* gv = reinterpret_cast<const unsigned char*>(v + head + (long long)kv * D);
    for (int ins = wu; ins < C::DMA_INS; ins += 4) {
      const int p = ins * 64 + lane, row = p / (C::NCH + 1), col = p % (C::NCH + 1);
      const int go = row * D * 2 + (col < C::NCH ? col : 0) * 16;
      __builtin_amdgcn_global_load_lds((gbl_void*)(gk + go), (lds_void*)(reinterpret_cast<unsigned char*>(sK) + ins * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void*)(gv + go), (lds_void*)(reinterpret_cast<unsigned char*>(sV) + ins * 1024), 16, 0, 0);
    }
  };
  if constexpr (C::PREFETCH) load_tile(0);
  for (int kv0 = 0; kv0 < kv_end; kv0 += C::BKV) {
    __syncthreads();  // every wave is done with the previous tile in LDS
    if constexpr (C::DMA) {
      dma_tile(kv0);  // complete at the barrier below (it waits for every vector-memory operation)
    } else {
      // the tile prefetched into registers during the previous one
#pragma unroll
      for (int x = 0; x < C::NPT; ++x) {
        const int cidx = tid + 256 * x, r = cidx / C::CPR, c = cidx % C::CPR;
        lds_store16(sK + r * C::P + 8 * c, kr[x]);
        lds_store16(sV + r * C::P + 8 * c, vr[x]);
      }
    }
    __syncthreads();
    if constexpr (C::PREFETCH) {
      if (kv0 + C::BKV < kv_end) load_tile(kv0 + C::BKV);  // in flight during this tile's products
    }
    if (CAUSAL && kv0 > q0 + 31) continue;  // whole tile masked for this wave

    // S^T = K Q^T : rows kv, columns q (lane)
    f32x16 sAcc[C::MK];
#pragma unroll
    for (int mb = 0; mb < C::MK; ++mb) sAcc[mb] = f32x16{};
#pragma unroll
    for (int s = 0; s < C::KD; ++s)
#pragma unroll
      for (int mb = 0; mb < C::MK; ++mb) sAcc[mb] = mfma32(frag_row(sK, C::P, 32 * mb, 16 * s), qB[s], sAcc[mb]);

    float mx = -INFINITY;
    // D = 128: mask only tiles that cross this wave's diagonal (D = 64 measured
    // faster masking every tile)
    const bool diag = CAUSAL && (D == 64 || kv0 + C::BKV - 1 > q0);
#pragma unroll
    for (int mb = 0; mb < C::MK; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = RAW_MAX ? sAcc[mb][r] : sAcc[mb][r] * c1;
        const int kv = kv0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (diag && kv > qi) x = -INFINITY;
        sAcc[mb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if constexpr (RAW_MAX) mx *= c1;  // -inf (a fully masked tile) stays -inf
    const float m_new = fmaxf(m_run, mx);  // finite: key 0 is visible to every query
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
    bf16x8 pB[C::KK];
#pragma unroll
    for (int mb = 0; mb < C::MK; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(RAW_MAX ? __builtin_fmaf(sAcc[mb][r], c1, -m_new) : sAcc[mb][r] - m_new);
        const __bf16 pb = (__bf16)p;
        lsum += p;
        pB[2 * mb + (r >> 3)][r & 7] = pb;
      }
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < C::ND; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oAcc[n][r] *= alpha;
    // O^T += V^T P^T : A = V^T (rows d, K = kv in the accumulator permutation), B = P^T
#pragma unroll
    for (int s = 0; s < C::KK; ++s)
#pragma unroll
      for (int n = 0; n < C::ND; ++n) oAcc[n] = mfma32(frag_tr(sV, C::P, 16 * s, 32 * n, true), pB[s], oAcc[n]);
  }

  const float inv = 1.f / l_run;
#pragma unroll
  for (int n = 0; n < C::ND; ++n)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * n + 8 * rq + 4 * g;
      bf16x4 v4 = to_bf16x4(oAcc[n][4 * rq] * inv, oAcc[n][4 * rq + 1] * inv, oAcc[n][4 * rq + 2] * inv,
                            oAcc[n][4 * rq + 3] * inv);
      *reinterpret_cast<bf16x4*>(o + head + (long long)qi * D + d0) = v4;
    }
  if (g == 0) lse[(long long)bh * S + qi] = (m_run + __log2f(l_run)) * 0.6931471805599453f;
}

}  // namespace detattn
