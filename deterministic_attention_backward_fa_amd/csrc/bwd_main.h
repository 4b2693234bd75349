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
// Accumulator initial values carry the row terms: the S product uses K_j
// scaled by scale*log2(e) (rounded to bf16 once per column) and its
// accumulator of row q starts at -LSE_q*log2(e), so P = exp2(acc) with no
// multiply per element; the dP accumulator starts at -D_q (so dS = P * acc).
// Causal masking sets the S initial value to -inf above the diagonal, on
// diagonal tiles only.
//
// Instruction streams of one tile (one wave runs per SIMD, so MFMA, VALU,
// LDS and memory work overlap only when interleaved in the wave's own stream):
//   top:   row terms of tile t as the accumulators' initial values (the
//          diagonal mask on diagonal tiles);
//   A:     S/dP MFMAs of row block 0, S/dP of block 1 with block 0's
//          elementwise work (exp2, dS, bf16 packing, dS^T stores) between
//          them, dV/dK of block 0 with block 1's elementwise work. Every MFMA's
//          LDS operand is read PF MFMAs ahead; the previous tile's dQ
//          contribution is published (flag += 1 per wave) once its writes have
//          landed; tile t+1's Q, dO and row terms are DMA'd (global_load_lds)
//          into the next of three buffers over the first half; the dQ tile's
//          flag is read near the end;
//   barrier (dS^T complete, tile t+1 in LDS): the one barrier of the tile;
//   B:     dQ partial MFMAs (dS^T from LDS, K^T from registers); if the turn
//          has come (flag >= 4 * rank), the accumulator is read under them,
//          else after a bounded wait; dV/dK MFMAs of the last row block, with
//          the accumulator writes spread among the first of them.
// dS^T alternates between two LDS buffers, so a wave may start stream A of
// tile t+1 while others still read tile t's dS^T. The accumulator is touched
// only through coherent accesses (agent scope, or workgroup scope plus an L1
// invalidate when a ring of workgroups shares one XCD's L2), so the hand-off
// needs no cache writeback: a wave's writes have landed once its vmcnt
// covers them, before it adds to the flag.
//
// LDS tiles of Q, dO, K, V are row-major with 16 bytes of padding per row and
// rows permuted inside 16-row blocks (rperm), which keeps both the row and the
// transposing fragment reads free of bank conflicts; dS^T is unpadded with an
// XOR swizzle of its 16-byte chunks. Every fragment address is one per-lane
// register plus a compile-time offset.
#pragma once
#include "common.h"
#include "tile_sched.h"

#include <type_traits>

// Scheduling parameters of the instruction streams (measured choices; the
// macros exist so variants can be compiled side by side):
//   PF         LDS operand loads run this many operands ahead of their MFMA
//   ELEM_DELAY MFMAs of a group issued before its first elementwise unit
//   DMA_SPAN   the next tile's DMA is spread over this fraction (1/8ths) of stream A
//   PUB_AT     stream-A MFMA of the next tile before which a wave publishes its
//              previous tile's dQ contribution
//   FLAG_AT    stream-A MFMA (in 1/8ths of stream A) before which the dQ tile's
//              flag is read, so its latency hides under the rest of stream A
//   DECIDE_AT  stream-B MFMA before which the flag value is examined (its
//              latency hides under the first dQ MFMAs) and the reads begin
//   LD_SPAN    the dQ accumulator reads are spread over this fraction (1/8ths)
//              of the dQ MFMAs (0: all before the first)
//   ST_AT, ST_SPAN  the accumulator writes start after this fraction (1/8ths)
//              of the dV/dK MFMAs of stream B and are spread over ST_SPAN 1/8ths
#ifndef DETATTN_PF
#define DETATTN_PF 4
#endif
#ifndef DETATTN_ELEM_DELAY
#define DETATTN_ELEM_DELAY 2
#endif
#ifndef DETATTN_DMA_SPAN
#define DETATTN_DMA_SPAN 4
#endif
#ifndef DETATTN_PUB_AT
#define DETATTN_PUB_AT 8
#endif
#ifndef DETATTN_FLAG_AT
#define DETATTN_FLAG_AT 7
#endif
#ifndef DETATTN_DECIDE_AT
#define DETATTN_DECIDE_AT 2
#endif
#ifndef DETATTN_LD_SPAN
#define DETATTN_LD_SPAN 7
#endif
#ifndef DETATTN_ST_AT
#define DETATTN_ST_AT 0
#endif
#ifndef DETATTN_ST_SPAN
#define DETATTN_ST_SPAN 8
#endif

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
  // dQ partial (BQ x D) split over the 4 waves: each wave owns DW 32-column
  // blocks x MQD 32-row blocks. Two column blocks per wave (when the tile has
  // enough blocks) let one dS operand read feed two MFMAs.
  static constexpr int DW = (ND >= 2 && ND * (BQ / 32) >= 8) ? 2 : 1;
  static constexpr int MQD = ND * (BQ / 32) / (4 * DW);
  static constexpr int DGRP = ND / DW;   // column-block groups
  static constexpr int NCH = D / 8;      // 16-byte chunks per Q/dO/K/V row
  static constexpr int PD = D * 2 + 16;  // padded row pitch of Q/dO/K/V tiles (bytes)
  static constexpr int NCH_S = BQ / 8;   // 16-byte chunks per dS^T row
  static constexpr int PS = BQ * 2;      // dS^T row pitch (bytes; XOR-swizzled chunks, see swz_f)
  static constexpr int QB = BQ * PD;     // one Q or dO tile
  static constexpr int KB = BKV * PD;    // one K or V tile
  static constexpr int SB = BKV * PS;    // dS^T tile (row kv, column q)
  static constexpr int LDB = BQ * 8;     // -LSE/scale then -D, fp32
  static constexpr int OFF_LD = 2 * QB;
  static constexpr int BUF = OFF_LD + LDB;  // one Q-tile buffer: Q, dO, row terms
  static constexpr int OFF_DS = 0;
  // Q-tile buffers: the next tile is loaded one tile ahead; the third buffer
  // gives K_j, V_j room to be staged at the start of a column next to the
  // first Q tile, and lets one barrier per tile suffice
  static constexpr int NBUF = 3;
  // Two dS^T buffers (alternating per tile, when LDS allows) let a wave start
  // the next tile's stream A while others still read this tile's dS^T, so a
  // tile needs one barrier (after stream A) instead of two.
  static constexpr int NDS = (2 * SB + NBUF * BUF + 16 <= 160 * 1024) ? 2 : 1;
  static constexpr int OFF_B0 = NDS * SB;  // buffer b at OFF_B0 + b * BUF
  // K_j, V_j are staged in buffers 1.. at the start of a column (they move to
  // registers before those buffers receive Q tiles)
  static constexpr int OFF_K = OFF_B0 + BUF;
  static constexpr int OFF_V = OFF_K + KB;
  static constexpr int TILE_END = OFF_B0 + NBUF * BUF;
  // Resident-pair variant of symmetric shift: the pair's second column K, V
  // are staged next to the first (both within the tile buffers)
  static constexpr int OFF_K2 = OFF_V + KB;
  static constexpr int OFF_V2 = OFF_K2 + KB;
  static constexpr bool PAIR_FITS = OFF_V2 + KB <= TILE_END;
  static constexpr int DMA_Q = BQ * (NCH + 1) / 64;  // 1 KB DMA instructions per padded Q/dO tile
  static constexpr int DMA_K = BKV * (NCH + 1) / 64;
  static constexpr int DMA_QW = (DMA_Q + 3) / 4;     // per wave, at most
  // DMA work of one wave for one Q tile, in slots issued one by one between
  // MFMAs: Q and dO rows, then the row terms
  static constexpr int DMA_SLOTS = 2 * DMA_QW + 1;
  // vector-memory instructions of DMA slot u (the row-term slot takes BQ / 64)
  static constexpr int slot_vmem(int u) { return u < 2 * DMA_QW ? 1 : BQ / 64; }
  // Epilogue scratch, aliasing the tile buffers (nothing is in flight then):
  // per output tensor, the fp32 partials of the waves with wq == 1 (NQW == 2)
  // and a padded bf16 tile for coalesced stores.
  static constexpr int PO = D + 8;
  static constexpr int RED_BYTES = (NQW == 2) ? NKVW * 32 * D * 4 : 0;
  static constexpr int OUT_BYTES = BKV * PO * 2;
  static constexpr int EPI_END = RED_BYTES + OUT_BYTES;
  static constexpr int OFF_MISC = TILE_END > EPI_END ? TILE_END : EPI_END;
  static constexpr int LDS_BYTES = OFF_MISC + 64;  // 16 ints: ticket, XCD registration
  static_assert(NKVW * NQW == 4, "4 waves");
  static_assert(QW % 32 == 0 && MQD >= 1 && DGRP * DW == ND && 4 * DW * MQD == ND * (BQ / 32), "tile shape");
  static_assert(MQD == 1, "one dS row block per wave (the swizzled dS reads use per-lane offsets)");
  static_assert((BQ * (NCH + 1)) % 64 == 0 && (BKV * (NCH + 1)) % 64 == 0, "DMA granularity");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(OFF_V + KB <= TILE_END, "K, V staging");
};

// Order of the MFMAs of stream A (before the dS^T barrier). Group gi holds the
// S/dP MFMAs of row block gi (gi < MQ) followed by the dV/dK MFMAs of row block
// gi - 2 (2 <= gi <= MQ); the elementwise work of block gi - 1 is spread over
// group gi. Each MFMA is identified by kind (0 S, 1 dP, 2 dV, 3 dK), row block
// and step (K step for S/dP; 0 .. 2*ND-1 over (Q K step, D block) for dV/dK).
template <class C>
struct StreamA {
  static constexpr int NSDP = 2 * C::KD;
  static constexpr int NDK = 4 * C::ND;
  static constexpr int gsize(int gi) { return (gi < C::MQ ? NSDP : 0) + (gi >= 2 && gi <= C::MQ ? NDK : 0); }
  static constexpr int gstart(int gi) {
    int s = 0;
    for (int x = 0; x < gi; ++x) s += gsize(x);
    return s;
  }
  static constexpr int N = gstart(C::MQ + 1);
  static constexpr int group(int k) {
    int gi = 0;
    while (gi < C::MQ && k >= gstart(gi + 1)) ++gi;
    return gi;
  }
  static constexpr int rel(int k) { return k - gstart(group(k)); }
  static constexpr bool sdp(int k) { return group(k) < C::MQ && rel(k) < NSDP; }
  static constexpr int drel(int k) { return rel(k) - (group(k) < C::MQ ? NSDP : 0); }
  static constexpr int kind(int k) { return sdp(k) ? (rel(k) & 1) : 2 + (drel(k) & 1); }
  static constexpr int blk(int k) { return sdp(k) ? group(k) : group(k) - 2; }
  static constexpr int step(int k) { return sdp(k) ? (rel(k) >> 1) : (drel(k) >> 1); }
  // LDS instructions of MFMA k's operand load, and those issued after it by
  // the time MFMA k runs (operands are loaded pf MFMAs ahead)
  static constexpr int nloads(int k) { return sdp(k) ? 1 : 2; }
  static constexpr int loads_after(int k, int pf) {
    int n = 0;
    for (int x = k + 1; x <= k + pf && x < N; ++x) n += nloads(x);
    return n;
  }
  // elementwise units (16 elements + 4 dS^T stores) issued after the j-th MFMA
  // of a group of size G: the first DELAY MFMAs of the group carry none, so
  // the previous group's last results have landed.
  // DMA slots of the next Q tile issued after MFMA k: spread evenly over the
  // stream from MFMA 1 on, so the texture path is never flooded
  static constexpr int dma_before(int k) {
    const int U = C::DMA_SLOTS, S0 = 1;
    const int E = S0 + 1 + ((N - S0 - 1) * DETATTN_DMA_SPAN) / 8;  // all slots issued by MFMA E
    if (k <= S0) return 0;
    if (k >= E) return U;
    const int v = ((k - S0) * U + (E - S0 - 1)) / (E - S0);
    return v < U ? v : U;
  }
  // vector-memory instructions the DMA slots issue before MFMA k
  static constexpr int dma_vmem_before(int k) {
    int n = 0;
    for (int u = 0; u < dma_before(k); ++u) n += C::slot_vmem(u);
    return n;
  }
  // the previous tile's contribution is published at the top of MFMA kPub
  static constexpr int kPub = DETATTN_PUB_AT < N ? DETATTN_PUB_AT : N - 1;
  static constexpr int kFlag = (N * DETATTN_FLAG_AT) / 8 < N ? (N * DETATTN_FLAG_AT) / 8 : N - 1;
  // the flag read is the last vector-memory operation of stream A
  static_assert(dma_before(kFlag) == C::DMA_SLOTS, "every DMA slot precedes the flag read");
  static_assert(kPub >= 0, "publish slot");
  static constexpr int kUnits = 20;
  static constexpr int kDelay = DETATTN_ELEM_DELAY;
  static constexpr int units_before(int j, int G) {
    return j <= kDelay ? 0 : (j >= G ? kUnits : ((j - kDelay) * kUnits) / (G - kDelay));
  }
};

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Order of the MFMAs of stream B (after the dS^T barrier): the dQ partial
// (KKV K steps x MQD row blocks x DW column blocks; one dS operand, read with
// two transposing reads, serves the DW column blocks), then the dV/dK MFMAs
// of the last row block (one operand each). Loads are numbered separately
// from MFMAs: MFMA k uses load load_of(k), and loads run pf loads ahead.
template <class C>
struct StreamB {
  static constexpr int NB1 = C::KKV * C::MQD * C::DW;  // dQ MFMAs
  static constexpr int N = NB1 + 4 * C::ND;
  static constexpr int NL1 = C::KKV * C::MQD;          // dQ operand loads
  static constexpr int NL = NL1 + 4 * C::ND;
  static constexpr int load_of(int k) { return k < NB1 ? k / C::DW : NL1 + (k - NB1); }
  static constexpr bool first_use(int k) { return k >= NB1 || k % C::DW == 0; }
  static constexpr int ninst(int) { return 2; }  // LDS instructions of a load (two transposing halves)
  // last load issued before MFMA k runs
  static constexpr int issued_by(int k, int pf) {
    const int x = load_of(k) + pf;
    return x < NL - 1 ? x : NL - 1;
  }
  static constexpr int insts_after(int k, int pf) {
    int n = 0;
    for (int l = load_of(k) + 1; l <= issued_by(k, pf); ++l) n += ninst(l);
    return n;
  }
};

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

#define DETATTN_FENCE() __builtin_amdgcn_sched_barrier(0)

// LDS operand loads of the MFMA streams are issued from inline assembly and
// waited for explicitly: the compiler would otherwise make every transposed
// read wait for all LDS-DMA transfers in flight (the next tile's prefetch).
// lgkm_wait<N> returns once at most N LDS operations are outstanding; the
// streams pass the number of their own loads issued after the awaited one, so
// any other LDS traffic can only make the wait longer, never too short. The
// awaited register is tied to the wait so the consuming MFMA stays after it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_ld16_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_ld16_agpr(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=a"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr_agpr(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=a"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& x) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
// the two halves of a transposed operand are tied to the wait before they are
// combined, so no copy of either half can run ahead of the data
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2& lo, u32x2& hi) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo), "+v"(hi) : "i"(N));
}
template <int N, class T>
__device__ __forceinline__ void lgkm_wait_agpr(T& x) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+a"(x) : "i"(N));
}
// one MFMA operand in flight: a 16-byte row read, or two transposed 8-byte reads
struct Opnd {
  u32x4 q;
  u32x2 lo, hi;
};
__device__ __forceinline__ u32x4 cat2(const u32x2& a, const u32x2& b) { return u32x4{a[0], a[1], b[0], b[1]}; }
// one wait for two operands (Q0/Q1: the operand is a 16-byte read, else two
// transposing halves); every register of both is tied to the wait
template <int N, bool Q0, bool Q1>
__device__ __forceinline__ void lgkm_wait2(Opnd& a, Opnd& b) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  if constexpr (Q0 && Q1)
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a.q), "+v"(b.q) : "i"(N));
  else if constexpr (Q0)
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a.q), "+v"(b.lo), "+v"(b.hi) : "i"(N));
  else if constexpr (Q1)
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a.lo), "+v"(a.hi), "+v"(b.q) : "i"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a.lo), "+v"(a.hi), "+v"(b.lo), "+v"(b.hi) : "i"(N));
}

// Workgroup barrier for LDS hand-offs only: LDS operations are complete, but
// vector-memory loads in flight (the prefetch DMA) stay in flight.
// (__syncthreads also waits for every outstanding vector-memory operation.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// 16-byte buffer read (per lane: voff + OFF bytes past the resource base plus
// soff), issued outside the compiler's wait tracking: the caller waits with
// vm_wait_tied. SC1 selects coherence across XCDs, else within the XCD (sc0).
template <int OFF, bool SC1>
__device__ __forceinline__ f32x4 buf_load16_asm(const u32x4& rsrc, uint32_t voff, uint32_t soff) {
  static_assert(OFF >= 0 && OFF < 4096, "buffer offset field");
  f32x4 r;
  if constexpr (SC1)
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4 sc1" : "=v"(r) : "v"(voff), "s"(rsrc), "s"(soff), "i"(OFF));
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4 sc0" : "=v"(r) : "v"(voff), "s"(rsrc), "s"(soff), "i"(OFF));
  return r;
}
// wait until at most N vector-memory operations are in flight; x is the
// register the awaited read filled (it is tied to the wait)
template <int N>
__device__ __forceinline__ void vm_wait_tied(f32x4& x) {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }
// keep a value in accumulation registers (AGPRs): MFMA-only operands live
// there, which leaves the VGPRs to the values the VALU works on
template <class T>
__device__ __forceinline__ void pin_agpr(T& x) {
  asm volatile("" : "+a"(x));
}
// dV/dK accumulation: an MFMA whose accumulator stays in AGPRs (the other
// MFMAs of the kernel are compiled in VGPR form, so the VALU reads S, dP and
// the dQ partial without copies). The compiler does not see these as MFMAs,
// so their hazards are covered by construction: the A operand (P or dS,
// written by the VALU) is produced at least one MFMA group earlier, the B
// operand arrives through lgkm_wait, consecutive uses of one accumulator are
// 2*ND - 1 MFMAs apart, and mfma_agpr_drain() runs before the VALU reads the
// accumulators.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// more wait states than an MFMA result needs before a VALU read
__device__ __forceinline__ void mfma_agpr_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
// keep a value in VGPRs (accumulators the VALU reads)
template <class T>
__device__ __forceinline__ void pin_vgpr(T& x) {
  asm volatile("" : "+v"(x));
}

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

// Q, dO, K, V tiles in LDS: rows padded by 16 bytes, and inside every 16-row
// block logical row r sits at physical row rperm(r) = 4*(r%4) + (r/4)%4 (an
// involution). With the 272-byte (D = 128) or 144-byte (D = 64) pitch each row
// starts 4 (or 36) banks after the previous one, so
//  * 16 consecutive logical rows read at one 16-byte column (row fragments)
//    cover all 64 banks once, and
//  * the four logical rows a 16-lane group reads transposed (4j + g .. for
//    rows 4g..4g+3) start 16 banks apart, each group's 32-byte reads of two
//    16-lane groups filling the 64 banks once;
// logical row r + 8 sits 2 physical rows after r, r + 4 one row after (for r
// with (r/4)%4 even), and multiples of 16 are unchanged, so those steps stay
// compile-time offsets.
__host__ __device__ constexpr int rperm(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// Global byte offset, inside a row-major tile of NCH-chunk rows, of the chunk
// that lane `lane` of DMA instruction `ins` moves into the padded, row-permuted
// LDS tile (NCH + 1 chunks per row). Padding chunks re-read chunk 0 of their
// row; those bytes land in the padding and are never read.
template <int NCH>
__device__ __forceinline__ int dma_goff(int ins, int lane) {
  const int p = ins * 64 + lane;
  const int row = p / (NCH + 1), col = p % (NCH + 1);
  return rperm(row) * (NCH * 16) + (col < NCH ? col : 0) * 16;
}

__device__ __forceinline__ void dma16(const void* gsrc, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void*)gsrc, (lds_void*)lds, 16, 0, 0);
}

// PAIR (symmetric shift only): both columns of a pair item keep their K, V
// and dK, dV in registers for the whole item (the pages' alternative to
// holding one column at a time), so the item has no column switch: the visits,
// the ranks and every result bit are those of the sequential form.
template <int D, int BQ, int BKV, bool CAUSAL, int DQM, bool TRACE, bool PAIR>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using C = MainCfg<D, BQ, BKV>;
  static_assert(!PAIR || C::PAIR_FITS, "pair K/V staging");
  constexpr int NSET = PAIR ? 2 : 1;  // register sets of K, V, K^T, dK, dV
  using SA = StreamA<C>;
  constexpr int PF = DETATTN_PF;  // LDS operand loads run this many MFMAs ahead
  constexpr int RING = PF + 2;  // operand registers; a slot is reloaded two MFMAs after its last reader
  // Scope of the accumulator accesses: across XCDs (sc1), or inside the XCD's
  // L2 (sc0) when every workgroup of a ring runs on one XCD. sc0 loads may hit
  // the compute unit's own L1, so that mode invalidates L1 (buffer_inv sc0)
  // after observing the flag and before loading. Flags always use sc1.
  constexpr bool kLocal = DQM == kDqLocalRmw || DQM == kDqUnorderedLocal;
  constexpr bool kUnordered = DQM == kDqUnordered || DQM == kDqUnorderedLocal;
  constexpr int kScope = kLocal ? __HIP_MEMORY_SCOPE_WORKGROUP : __HIP_MEMORY_SCOPE_AGENT;
  constexpr int kFlagScope = __HIP_MEMORY_SCOPE_AGENT;
  constexpr bool kRmw = DQM == kDqOrderedRmw || DQM == kDqLocalRmw;
  constexpr int kWaves = kThreads / 64;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  int* sMisc = reinterpret_cast<int*>(smem + C::OFF_MISC);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int s16 = lane & 15;
  const int grp = lane >> 4;
  const int wk = w % C::NKVW;
  const int wq = w / C::NKVW;
  const int nbq = (w % C::DGRP) * C::DW;    // dQ: this wave's first D block
  const int mq0 = (w / C::DGRP) * C::MQD;  // dQ: first 32-row block
  const float c1 = a.scale * kLog2e;  // K scale of the S product (exp2 domain)
  const Sched sc = a.sc;
  const int ipH = sc.items_per_head();
  const long long total_items = (long long)a.BH * ipH;

  // Per-lane LDS byte offsets; everything else in a fragment address is a
  // compile-time offset (or the per-tile buffer base).
  const int trcol = (16 * (grp & 1) + 4 * (s16 & 3)) * 2;
  // Q/dO row fragments (buffer-relative): logical row QW*wq + lane%32
  const int oA = rperm(C::QW * wq + c32) * C::PD + g * 16;
  // Q/dO transposed fragments in accumulator K order: logical rows 4g + j
  // (j = lane%16 / 4) at physical 4j + g; rows + 8 at physical + 2
  const int oT = (C::QW * wq + 4 * (s16 >> 2) + g) * C::PD + trcol;
  // dS^T (row kv, column q; chunk c of row r at c ^ swz_f(r)): transposed
  // fragments of the dQ product read rows 8g + j (lo) and 8g + j + 4 (hi)
  const int sq_chunk = 4 * mq0 + 2 * (grp & 1) + ((s16 & 3) >> 1);
  const int sr_lo = 8 * g + (s16 >> 2), sr_hi = sr_lo + 4;
  const int oS = C::OFF_DS + sr_lo * C::PS + ((sq_chunk ^ swz_f<C::NCH_S>(sr_lo)) << 4) + (s16 & 1) * 8;
  const int oS_hi = C::OFF_DS + sr_hi * C::PS + ((sq_chunk ^ swz_f<C::NCH_S>(sr_hi)) << 4) + (s16 & 1) * 8;
  // dS^T stores: row 32*wk + lane%32, chunk (QW*wq + 16 sq + 8 hh) / 8, bytes 8g
  const int w_row = 32 * wk + c32;
  const int w_swz = swz_f<C::NCH_S>(w_row);
  const int oW = C::OFF_DS + w_row * C::PS + 8 * g;
  const int oL = C::OFF_LD + (C::QW * wq + 4 * g) * 4;                           // row terms (buffer-relative)
  // dQ accumulator, fragment order: 32 x 32 blocks of 4 KB; inside a block,
  // register group h (rows 8h + 4g .. + 3, column lane%32) of every lane is
  // one 1 KB run, lane-major, 16 bytes per lane. A wave's block mb starts at
  // byte dqblk(mb) of the Q tile.
  constexpr int NQB = C::MQD * C::DW;  // dQ blocks of this wave: row block m, column block n at m * DW + n
  auto dqblk = [&](int mb) -> int { return ((mq0 + mb / C::DW) * C::ND + nbq + mb % C::DW) * 4096; };
  int dqlane[NQB];
#pragma unroll
  for (int mb = 0; mb < NQB; ++mb) dqlane[mb] = dqblk(mb) + lane * 16;
  // The atomic modes keep the accumulator row-major instead (their per-element
  // atomics then touch two 128-byte lines per instruction, not eight): lane
  // offset of row 32 mq0 + 4g, column 32 nbq + lane%32
  const int dqlane_rm = ((32 * mq0 + 4 * g) * D + 32 * nbq + c32) * 4;
  int goffQ[C::DMA_QW];
#pragma unroll
  for (int x = 0; x < C::DMA_QW; ++x) goffQ[x] = dma_goff<C::NCH>(w + 4 * x, lane);

  // Optional phase trace: wave 0, lane 0 of each workgroup.
  int trace_n = 0;
  auto trace_at = [&](int phase, int t, long long item, unsigned long long when) {
    if constexpr (TRACE) {
      if (tid == 0 && trace_n < a.trace_records) {
        unsigned long long* p = a.trace + ((size_t)blockIdx.x * a.trace_records + trace_n) * 2;
        p[0] = when;
        p[1] = (unsigned long long)phase | ((unsigned long long)(t & 0xFFFFFF) << 8) | ((unsigned long long)item << 32);
        ++trace_n;
      }
    }
  };
  auto trace_rec = [&](int phase, int t, long long item) {
    if constexpr (TRACE) trace_at(phase, t, item, __builtin_amdgcn_s_memtime());
  };
  // the workgroup's start, recorded once the ring set-up is done
  const unsigned long long t_start = TRACE ? __builtin_amdgcn_s_memtime() : 0ull;

  // Ring membership. Workgroup w is placed by a static map that assumes it
  // runs on XCD w % 8 (ring (u / G) * 8 + w % 8, slot u % G, u = w / 8): the
  // hardware's round-robin dispatch, which keeps each ring on one XCD.
  // In the XCD-local dQ modes (read-modify-write and atomics kept in one XCD's
  // L2) correctness needs that placement, so there every workgroup also
  // registers the XCD the hardware reports (a table entry per workgroup, set
  // when it arrives; the grid is co-resident), starts
  // loading its first item under the static map, and before the item's first
  // tile checks the registered placement: rings are formed per XCD from its
  // registered workgroups in index order (floor(count / G) rings per XCD,
  // numbered round-major over the XCDs), which under round-robin dispatch is
  // the static map. Only if the two differ does the workgroup drop what it
  // loaded and start over with the registered ring, so the result never
  // depends on how workgroups were dispatched, and the registration wait
  // overlaps the first K/V load.
  int ring_id = 0, slot = 0, n_rings = a.rings;
  bool confirm = false;  // the registered placement is still to be checked
  unsigned my_xcc = 0;
  if (!a.ticket_mode) {
    const int wg = blockIdx.x;
    // the static map's guess (testing: shifted by one workgroup, so that the
    // registered placement differs and every workgroup takes the restart path)
    const int wg_map = (kLocal && a.xcd_remap && a.misplace) ? (wg + 1) % (int)gridDim.x : wg;
    if (a.xcd_remap) {
      const int x = wg_map & 7, u = wg_map >> 3;
      ring_id = (u / a.ring) * 8 + x;
      slot = u % a.ring;
    } else {
      ring_id = wg / a.ring;
      slot = wg % a.ring;
    }
    if (kLocal && a.xcd_remap) {
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(my_xcc));
      my_xcc &= 7;
      // the workgroup's table entry is its arrival (the preprocess cleared the
      // table): a relaxed device-scope store, no counter that every workgroup
      // would update in turn
      if (tid == 0) __hip_atomic_store(a.xcd_tab + wg, my_xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      confirm = true;
    } else if (ring_id >= n_rings) {
      return;
    }
  }
  if (!confirm) trace_at(8, 0, 0, t_start);

  // The registered placement of this workgroup (XCD-local modes; every thread
  // takes part): waits until every workgroup has registered (bounded), then
  // sets ring_id, slot (ring_id = -1: no ring, or the wait timed out) and
  // n_rings from the table; returns whether they equal the static map's.
  auto registered_ring = [&]() -> bool {
    int* sCnt = sMisc + 4;  // 8 per-XCD counts, then this workgroup's rank on its XCD
    if (tid < 9) sCnt[tid] = 0;
    __syncthreads();
    if (w == 0) {
      // wave 0 reads the whole table (up to 16 entries per lane, all in
      // flight at once) until every entry is set, then counts from those values
      constexpr int NV = (int)WsLayout::kMaxXcdGrid / 64;
      const int G = (int)gridDim.x;
      unsigned v[NV];
      const long long t0 = now_ticks();
      int ok = 1;
      for (;;) {
        bool missing = false;
#pragma unroll
        for (int x = 0; x < NV; ++x) {
          const int w2 = lane + 64 * x;
          v[x] = w2 < G ? __hip_atomic_load(a.xcd_tab + w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1u;
          missing |= v[x] == 0u;
        }
        if (__builtin_amdgcn_ballot_w64(missing) == 0) break;
        __builtin_amdgcn_s_sleep(1);
        if (now_ticks() - t0 > a.timeout_ticks ||
            __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          if (lane == 0) report_error(a, kErrTimeout);
          ok = 0;
          break;
        }
      }
      if (ok) {
#pragma unroll
        for (int x = 0; x < NV; ++x) {
          const int w2 = lane + 64 * x;
          const int x2 = (int)v[x] - 1;
          if (w2 < G && x2 >= 0 && x2 < 8) {
            atomicAdd(sCnt + x2, 1);
            if (x2 == (int)my_xcc && w2 < (int)blockIdx.x) atomicAdd(sCnt + 8, 1);
          }
        }
      }
      if (lane == 0) sMisc[1] = ok;
    }
    __syncthreads();
    const bool ok = __builtin_amdgcn_readfirstlane(sMisc[1]) != 0;
    const int prev_ring = ring_id, prev_slot = slot, prev_n = n_rings;
    ring_id = -1;
    n_rings = 0;
    if (ok) {
      const int rank = __builtin_amdgcn_readfirstlane(sCnt[8]);
      const int k = rank / a.ring;
      int rid = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int rx = __builtin_amdgcn_readfirstlane(sCnt[x]) / a.ring;
        n_rings += rx;
        rid += (rx < k ? rx : k) + ((x < (int)my_xcc && rx > k) ? 1 : 0);
      }
      slot = rank % a.ring;
      if (k < __builtin_amdgcn_readfirstlane(sCnt[my_xcc]) / a.ring) ring_id = rid;
    }
    __syncthreads();  // the counts are read before anyone reuses them
    trace_at(8, 0, 0, t_start);
    trace_rec(9, slot, ring_id);  // registered: ring and slot known
    return ring_id == prev_ring && slot == prev_slot && n_rings == prev_n;
  };

  const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)smem;
  const uint32_t aS = lbase + oS, aS_hi = lbase + oS_hi;

  // Q, dO and the row terms of Q tile i -> buffer b (asynchronous).
  auto dma_q = [&](int b, long long head_off, long long bhS, int i) {
    const long long qrow0 = (long long)i * BQ;
    unsigned char* base = smem + C::OFF_B0 + b * C::BUF;
    const unsigned char* gq = reinterpret_cast<const unsigned char*>(a.q + head_off + qrow0 * D);
    const unsigned char* gd = reinterpret_cast<const unsigned char*>(a.dout + head_off + qrow0 * D);
    // goffQ[x] < 2^31: tile-relative byte offsets (uniform base + 32-bit offset addressing)
#pragma unroll
    for (int x = 0; x < C::DMA_QW; ++x) {
      const int ins = w + 4 * x;
      if (ins < C::DMA_Q) {
        dma16(gq + (uint32_t)goffQ[x], base + ins * 1024);
        dma16(gd + (uint32_t)goffQ[x], base + C::QB + ins * 1024);
      }
    }
    float* ld = reinterpret_cast<float*>(base + C::OFF_LD);
    dma_f32(ld, a.nlse + bhS + qrow0, BQ, 0);
    dma_f32(ld + BQ, a.ndelta + bhS + qrow0, BQ, 1);
  };

  // Ring mode: the ring takes heads ring_id, ring_id + rings, ...; inside a
  // head, workgroup `slot` takes one item per round of G = a.ring items: item
  // kG + slot in round k.
  // In snake order (a.snake) odd rounds hand the slots out in reverse, so a
  // workgroup whose items shrink with j (descending, causal mask) gets a
  // short item after a long one.
  int ring_bh = ring_id, ring_k0 = 0;
  bool ring_rev = false;
  for (;;) {
    long long gidx = -1;  // no item left
    if (a.ticket_mode) {
      if (tid == 0) sMisc[0] = (int)atomicAdd(a.ticket, 1u);
      __syncthreads();
      gidx = __builtin_amdgcn_readfirstlane(sMisc[0]);
      __syncthreads();
      if (gidx >= total_items) return;
    } else if (ring_id >= 0 && ring_id < n_rings && ring_bh < a.BH) {
      gidx = (long long)ring_bh * ipH + ring_k0 + (ring_rev ? a.ring - 1 - slot : slot);
      ring_k0 += a.ring;
      ring_rev = a.snake && !ring_rev;
      if (ring_k0 >= ipH) {
        ring_k0 = 0;
        ring_rev = false;
        ring_bh += n_rings;
      }
    }
    // The ticket counter hands out the ordered schedules' items head-major, the
    // greedy (head, KV tile) dispatch of the pages' DAG model. The unordered
    // reference takes them item-major over the heads (every head's item 0,
    // then every head's item 1, ...): under a causal mask its items shrink with
    // the KV tile, so the longest go first across all heads. Rings: head-major.
    int bh = 0, it = 0;
    if (gidx >= 0) {
      if (kUnordered && a.ticket_mode) {
        it = (int)(gidx / a.BH);
        bh = (int)(gidx % a.BH);
      } else {
        bh = (int)(gidx / ipH);
        it = (int)(gidx % ipH);
      }
    }
    const long long head_off = (long long)bh * a.S * D;
    const long long bhS = (long long)bh * a.S;
    // the head's dQ accumulator as a buffer resource (32-bit offsets, range-checked)
    const __amdgpu_buffer_rsrc_t dqrsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.dqacc + head_off, 0, a.S * D * 4, kBufferWord3);


    // K_j, V_j into their LDS tiles (asynchronous)
    auto dma_kv = [&](long long kv_head, int kv_j, int off_k = C::OFF_K) {
      const unsigned char* gk = reinterpret_cast<const unsigned char*>(a.k + kv_head + (long long)kv_j * BKV * D);
      const unsigned char* gv = reinterpret_cast<const unsigned char*>(a.v + kv_head + (long long)kv_j * BKV * D);
      for (int ins = w; ins < C::DMA_K; ins += 4) {
        const int go = dma_goff<C::NCH>(ins, lane);
        dma16(gk + go, smem + off_k + ins * 1024);
        dma16(gv + go, smem + off_k + (C::OFF_V - C::OFF_K) + ins * 1024);
      }
    };
    // The second column's K, V load while the first column's dK, dV go out
    // (the epilogue's LDS staging lies below the K, V tiles).
    static_assert(C::EPI_END <= C::OFF_K, "epilogue LDS overlaps the K/V tiles");

    // XCD-local rings: the registered placement is checked once, with the first
    // item's K, V and first Q tile already on their way
    bool first_loaded = false;
    if (confirm) {
      confirm = false;
      if (gidx >= 0) {
        int j0;
        const SegWalk w0 = sc.walk(it, 0, j0);
        dma_kv(head_off, j0);
        if constexpr (PAIR) dma_kv(head_off, sc.seg_kv(it, 1), C::OFF_K2);
        dma_q(0, head_off, bhS, w0.i);
      }
      if (!registered_ring()) {
        // placed otherwise than the static map assumed: drop what was loaded, take the registered ring
        if (gidx >= 0) {
          wait_vm_all();
          __syncthreads();
        }
        ring_bh = ring_id;
        ring_k0 = 0;
        ring_rev = false;
        continue;
      }
      first_loaded = gidx >= 0;
    }
    if (gidx < 0) return;

    // the resident pair's two register sets (the one-column form declares its
    // set inside the segment body, live for that column only)
    bf16x8 kB_[NSET][C::KD], vB_[NSET][C::KD], kTB_[NSET][C::KKV * C::DW];
    f32x16 dKacc_[NSET][C::ND], dVacc_[NSET][C::ND];
    // K_j, V_j (MFMA B operands of S, dP) and K_j transposed (B operand of the
    // dQ partial) from their LDS staging (at off_k) straight into AGPRs
    auto load_kv_regs = [&](bf16x8(&kB)[C::KD], bf16x8(&vB)[C::KD], bf16x8(&kTB)[C::KKV * C::DW], int off_k) {
      const uint32_t ak = lbase + off_k + rperm(32 * wk + c32) * C::PD + g * 16;
      const uint32_t av = ak + (C::OFF_V - C::OFF_K);
      // K transposed (non-permuted K order): logical rows 8g + j at physical 4j + 2g, rows + 4 at + 1
      const uint32_t akt = lbase + off_k + (4 * (s16 >> 2) + 2 * g) * C::PD + trcol + 64 * nbq;
      constexpr int NT = C::KKV * C::DW;  // K^T fragments: K step s, column block n at s * DW + n
      u32x4 kq[C::KD], vq[C::KD];
      u32x2 tlo[NT], thi[NT];
      static_for<0, C::KD>([&](auto sc_) {
        constexpr int s = decltype(sc_)::value;
        kq[s] = lds_ld16_asm<32 * s>(ak);  // scaled below, then moved to AGPRs
        vq[s] = lds_ld16_agpr<32 * s>(av);
      });
      static_for<0, NT>([&](auto xc) {
        constexpr int x = decltype(xc)::value, s = x / C::DW, n = x % C::DW;
        tlo[x] = lds_tr_agpr<16 * s * C::PD + 64 * n>(akt);
        thi[x] = lds_tr_agpr<(16 * s + 1) * C::PD + 64 * n>(akt);
      });
      // every loaded register is tied to a wait that covers it (loads complete in order)
      static_for<0, C::KD>([&](auto sc_) {
        constexpr int s = decltype(sc_)::value;
        constexpr int after_k = 2 * (C::KD - 1 - s) + 1 + 2 * NT;
        lgkm_wait<cmin(after_k, 15)>(kq[s]);  // more loads than the counter holds: 15 is still safe
        lgkm_wait_agpr<cmin(after_k - 1, 15)>(vq[s]);
      });
      static_for<0, NT>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        constexpr int after_t = 2 * (NT - 1 - x);
        lgkm_wait_agpr<cmin(after_t + 1, 15)>(tlo[x]);
        lgkm_wait_agpr<cmin(after_t, 15)>(thi[x]);
      });
#pragma unroll
      for (int s = 0; s < C::KD; ++s) {
        // K_j * scale * log2(e), rounded to bf16 (RNE): the S accumulator is then
        // directly the exp2 argument
        const bf16x8 kraw = as_bf16x8(kq[s]);
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const bf16x2 p2 = cvt2((float)kraw[t] * c1, (float)kraw[t + 1] * c1);
          kB[s][t] = p2[0];
          kB[s][t + 1] = p2[1];
        }
        vB[s] = as_bf16x8(vq[s]);
        pin_agpr(kB[s]);
        pin_agpr(vB[s]);
      }
#pragma unroll
      for (int x = 0; x < NT; ++x) {
        kTB[x] = as_bf16x8(cat2(tlo[x], thi[x]));
        pin_agpr(kTB[x]);
      }
    };
    auto zero_acc = [&](f32x16(&dK)[C::ND], f32x16(&dV)[C::ND]) {
#pragma unroll
      for (int n = 0; n < C::ND; ++n) {
        dK[n] = f32x16{};
        dV[n] = f32x16{};
        pin_agpr(dK[n]);
        pin_agpr(dV[n]);
      }
    };

    auto seg_body = [&](auto setc, int seg) {
    constexpr int SET = decltype(setc)::value;
    bf16x8 kB_col[C::KD], vB_col[C::KD], kTB_col[C::KKV * C::DW];
    f32x16 dK_col[C::ND], dV_col[C::ND];
    bf16x8(&kB)[C::KD] = PAIR ? kB_[SET] : kB_col;
    bf16x8(&vB)[C::KD] = PAIR ? vB_[SET] : vB_col;
    bf16x8(&kTB)[C::KKV * C::DW] = PAIR ? kTB_[SET] : kTB_col;
    f32x16(&dKacc)[C::ND] = PAIR ? dKacc_[SET] : dK_col;
    f32x16(&dVacc)[C::ND] = PAIR ? dVacc_[SET] : dV_col;
    const int t_begin = sc.seg_begin(it, seg), t_end = sc.seg_end(it, seg);
    int j;
    SegWalk cur = sc.walk(it, seg, j);  // at step t_begin
    const int i0 = cur.i;
    // ---- segment prologue: K_j, V_j (the second column of a symmetric pair has
    // them on their way already) and the first Q tile ----
    if (!first_loaded) {
      if (seg == 0) {
        dma_kv(head_off, j);
        if constexpr (PAIR) dma_kv(head_off, sc.seg_kv(it, 1), C::OFF_K2);
      }
      dma_q(0, head_off, bhS, i0);
    }
    first_loaded = false;
    wait_vm_all();
    __syncthreads();
    if constexpr (PAIR) {
      // the pair's two columns enter registers at the item's start
      if constexpr (SET == 0) {
        load_kv_regs(kB_[0], vB_[0], kTB_[0], C::OFF_K);
        load_kv_regs(kB_[1], vB_[1], kTB_[1], C::OFF_K2);
        zero_acc(dKacc_[0], dVacc_[0]);
        zero_acc(dKacc_[1], dVacc_[1]);
      }
    } else {
      load_kv_regs(kB, vB, kTB, C::OFF_K);
      zero_acc(dKacc, dVacc);
    }
    // K, V are in registers: buffer 1 is free for the next Q tile
    lds_barrier();
    trace_rec(6, t_begin, gidx);

    int t = t_begin;
    int* pend = nullptr;  // flag of the previous tile's contribution, not yet published
    int b = 0;    // buffer of tile t
    int dsb = 0;  // byte offset of tile t's dS^T buffer
    do {
      const int i = cur.i;
      const int nb = b + 1 == C::NBUF ? 0 : b + 1;  // buffer of tile t+1
      const long long qrow0 = (long long)i * BQ;
      trace_rec(0, t, gidx);
      // The next tile of this column goes into the other buffer; its DMA is
      // issued slot by slot during stream A, without branches: a wave with
      // fewer instructions than others repeats its tile's last instruction,
      // and in the last tile of a column the current tile is loaded again
      // into the idle buffer (the same bytes, or bytes no one reads).
      SegWalk nxt = cur;
      if (t + 1 < t_end) nxt.advance(t + 1);
      const int ni = __builtin_amdgcn_readfirstlane(nxt.i);
      const long long nrow0 = (long long)ni * BQ;
      unsigned char* nbase = smem + C::OFF_B0 + nb * C::BUF;
      auto dma_slot = [&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u < 2 * C::DMA_QW) {
          constexpr int x = u / 2;
          const int ins = w + 4 * x < C::DMA_Q ? w + 4 * x : C::DMA_Q - 1;
          const int go = w + 4 * x < C::DMA_Q ? goffQ[x] : dma_goff<C::NCH>(C::DMA_Q - 1, lane);
          const __bf16* src = (u & 1) ? a.dout : a.q;
          dma16(reinterpret_cast<const unsigned char*>(src + head_off + nrow0 * D) + (uint32_t)go,
                nbase + ((u & 1) ? C::QB : 0) + ins * 1024);
        } else {
          // row terms: waves 0, 2 load -LSE/scale, waves 1, 3 load -D (duplicates write the same bytes)
          float* ld = reinterpret_cast<float*>(nbase + C::OFF_LD) + (w & 1) * BQ;
          const float* src = ((w & 1) ? a.ndelta : a.nlse) + bhS + nrow0;
#pragma unroll
          for (int x = 0; x < BQ; x += 64)
            __builtin_amdgcn_global_load_lds((gbl_void*)(src + x + lane), (lds_void*)(ld + x), 4, 0, 0);
        }
      };
      // this tile's turn in dQ tile i's order: rank rk; the flag counts the wave contributions added
      const int rk = kUnordered ? 0 : cur.rank_now();
      int* flag = a.flags + ((long long)bh * sc.n_q + i) * kFlagInts;
      int seen = rk;  // the flag as last read (read in stream A)
      const int vb = C::OFF_B0 + b * C::BUF;
      const int vL = oL + vb;
      const uint32_t aA = lbase + oA + vb, aT = lbase + oT + vb;

      // ---- accumulator initial values: -LSE*log2(e) (S), -D (dP); mask on diagonal tiles ----
      f32x16 sAcc[C::MQ], pAcc[C::MQ];
#pragma unroll
      for (int m = 0; m < C::MQ; ++m)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(smem + vL + (32 * m + 8 * rq) * 4);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(smem + vL + BQ * 4 + (32 * m + 8 * rq) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sAcc[m][4 * rq + e] = l4[e];
            pAcc[m][4 * rq + e] = d4[e];
          }
        }
#pragma unroll
      for (int m = 0; m < C::MQ; ++m) {
        pin_vgpr(sAcc[m]);
        pin_vgpr(pAcc[m]);
      }
      if (CAUSAL && (long long)(j + 1) * BKV - 1 > qrow0) {
        // key index minus query index, both relative to the tile's first Q row
        const int kv_rel = (int)((long long)j * BKV - qrow0) + 32 * wk + c32 - C::QW * wq - 4 * g;
#pragma unroll
        for (int m = 0; m < C::MQ; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kv_rel > 32 * m + 8 * (r >> 2) + (r & 3)) sAcc[m][r] = -__builtin_inff();
      }

      bf16x8 pB[C::KQ], dsB[C::KQ];
      float pv[16], dv[16];
      Opnd ring[RING];

      // LDS operand of stream-A MFMA k (S, dP: one row read; dV, dK: two transposed reads)
      auto loadA = [&](auto kc, Opnd& o) {
        constexpr int k = decltype(kc)::value;
        constexpr int kind = SA::kind(k), m = SA::blk(k), st = SA::step(k);
        if constexpr (kind == 0) o.q = lds_ld16_asm<32 * m * C::PD + 32 * st>(aA);
        else if constexpr (kind == 1) o.q = lds_ld16_asm<C::QB + 32 * m * C::PD + 32 * st>(aA);
        else {
          constexpr int sq = 2 * m + st / C::ND, n = st % C::ND;
          constexpr int off = (kind == 2 ? C::QB : 0) + 16 * sq * C::PD + 64 * n;
          o.lo = lds_tr_asm<off>(aT);
          o.hi = lds_tr_asm<off + 2 * C::PD>(aT);
        }
      };
      // wait for MFMA k's operand (N = own loads issued after it) and return it
      auto waitA = [&](auto kc, Opnd& o) -> u32x4 {
        constexpr int k = decltype(kc)::value;
        constexpr int N = SA::loads_after(k, PF);
        if constexpr (SA::sdp(k)) {
          lgkm_wait<N>(o.q);
          return o.q;
        } else {
          lgkm_wait<N>(o.lo, o.hi);
          return cat2(o.lo, o.hi);
        }
      };
      auto mfmaA = [&](auto kc, const u32x4& opr) {
        constexpr int k = decltype(kc)::value;
        constexpr int kind = SA::kind(k), m = SA::blk(k), st = SA::step(k);
        const bf16x8 op = as_bf16x8(opr);
        if constexpr (kind == 0) sAcc[m] = mfma32(op, kB[st], sAcc[m]);
        else if constexpr (kind == 1) pAcc[m] = mfma32(op, vB[st], pAcc[m]);
        else {
          constexpr int sq = 2 * m + st / C::ND, n = st % C::ND;
          if constexpr (kind == 2) mfma_agpr(dVacc[n], pB[sq], opr);
          else mfma_agpr(dKacc[n], dsB[sq], opr);
        }
      };
      // elementwise unit u of row block e: 4 elements then one dS^T store, x4
      auto unitA = [&](auto ec, auto uc) {
        constexpr int e = decltype(ec)::value, u = decltype(uc)::value;
        constexpr int q4 = u / 5, pos = u % 5;
        if constexpr (pos < 4) {
          constexpr int r = 4 * q4 + pos;
          pv[r] = __builtin_amdgcn_exp2f(sAcc[e][r]);
          dv[r] = pv[r] * pAcc[e][r];
          if constexpr (r & 1) {
            constexpr int sq = 2 * e + (r >> 3), sl = (r - 1) & 7;
            const bf16x2 p2 = cvt2(pv[r - 1], pv[r]);
            const bf16x2 d2 = cvt2(dv[r - 1], dv[r]);
            pB[sq][sl] = p2[0];
            pB[sq][sl + 1] = p2[1];
            dsB[sq][sl] = d2[0];
            dsB[sq][sl + 1] = d2[1];
          }
        } else {
          // rows 4*q4 .. 4*q4+3 of the block: Q K step 2e + q4/2, half q4 & 1
          constexpr int sq = 2 * e + (q4 >> 1), hh = q4 & 1;
          bf16x4 v4;
#pragma unroll
          for (int x = 0; x < 4; ++x) v4[x] = dsB[sq][4 * hh + x];
          const int chunk = (C::QW * wq) / 8 + 2 * sq + hh;
          *reinterpret_cast<bf16x4*>(smem + dsb + oW + ((chunk ^ w_swz) << 4)) = v4;
        }
      };

      // ---- stream A ----
      static_for<0, PF>([&](auto kc) {
        if constexpr (decltype(kc)::value < SA::N) loadA(kc, ring[decltype(kc)::value]);
      });
      static_for<0, SA::N>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (!kUnordered && k == SA::kPub) {
          // publish the previous tile's contribution once its writes have
          // landed: only this tile's DMA was issued after them, and vector
          // memory operations complete in issue order
          if (pend != nullptr) {
            vm_wait<SA::dma_vmem_before(k)>();
            if (lane == 0) __hip_atomic_fetch_add(pend, 1, __ATOMIC_RELAXED, kFlagScope);
            pend = nullptr;
          }
        }
        if constexpr (!kUnordered && k == SA::kFlag) {
          // the dQ tile's flag, read late in stream A (every lane reads the
          // same word; also by the first contributor, so this read is always
          // the wave's newest vector-memory operation at the barrier); it is
          // re-polled after the dQ MFMAs only if the turn had not come
          seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, kFlagScope);
        }
        if constexpr (k + PF < SA::N) loadA(std::integral_constant<int, k + PF>{}, ring[(k + PF) % RING]);
        // operands are awaited in pairs: the even MFMA's wait also covers the
        // next one, which then needs neither a wait nor a hazard gap
        constexpr bool q0 = SA::sdp(k);
        if constexpr (k % 2 == 0 && k + 1 < SA::N) {
          constexpr bool q1 = SA::sdp(k + 1);
          lgkm_wait2<SA::loads_after(k + 1, PF - 1), q0, q1>(ring[k % RING], ring[(k + 1) % RING]);
          mfmaA(kc, q0 ? ring[k % RING].q : cat2(ring[k % RING].lo, ring[k % RING].hi));
        } else if constexpr (k % 2 == 1) {
          mfmaA(kc, q0 ? ring[k % RING].q : cat2(ring[k % RING].lo, ring[k % RING].hi));
        } else {
          mfmaA(kc, waitA(kc, ring[k % RING]));
        }
        DETATTN_FENCE();
        static_for<SA::dma_before(k), SA::dma_before(k + 1)>([&](auto uc) { dma_slot(uc); });
        constexpr int gi = SA::group(k);
        if constexpr (gi >= 1) {
          constexpr int G = SA::gsize(gi), jx = k - SA::gstart(gi);
          constexpr int u0 = SA::units_before(jx, G), u1 = SA::units_before(jx + 1, G);
          static_for<u0, u1>([&](auto uc) { unitA(std::integral_constant<int, gi - 1>{}, uc); });
        }
        DETATTN_FENCE();
      });
      if constexpr (SA::gsize(C::MQ) == 0)  // one row block: its elementwise work has no MFMAs to hide under
        static_for<0, SA::kUnits>([&](auto uc) { unitA(std::integral_constant<int, C::MQ - 1>{}, uc); });
      trace_rec(1, t, gidx);
      // this wave's share of the next tile (DMA issued early in stream A) has
      // landed: after the barrier below the whole next tile is in LDS. The
      // flag read, issued after it, may stay in flight.
      vm_wait<!kUnordered ? 1 : 0>();

      // The turn has come once every wave of every earlier contributor has
      // added: flag >= kWaves * rk. The counter only grows, and a wave of this
      // workgroup adds only after seeing the turn, so a larger value (a
      // sibling wave already done) also means the turn has come.
      const int turn_val = kWaves * rk;
      lds_barrier();  // dS^T complete
      // early (decided at stream-B MFMA kDecide): the turn has come already (or
      // this is the first contribution), so the accumulator is read right away
      // and the adds are issued early; the delay injection of the tests always
      // takes the late path
      bool early = false;

      // ---- stream B: dQ partial = dS K (this wave's DW column blocks x MQD row blocks), then dV/dK of the last block ----
      using SB_ = StreamB<C>;
      constexpr int NB1 = SB_::NB1;
      constexpr int NB = SB_::N;
      // atomic modes: MFMA index at which the adds count as issued (trace)
      constexpr int kAddLate = NB1 + (3 * SA::NDK) / 4;
      // RMW: the NLD 16-byte reads per lane go out under the dQ MFMAs, the
      // writes under the dV/dK MFMAs, spread so the vector-memory path takes
      // no burst
      constexpr int NLD = NQB * 4;
      constexpr int kDecide = DETATTN_DECIDE_AT < NB1 ? DETATTN_DECIDE_AT : 0;
      constexpr int kStBegin = NB1 + ((NB - NB1) * DETATTN_ST_AT) / 8;
      auto ld_at = [](int x) constexpr { return kDecide + (x * (((NB1 - kDecide) * DETATTN_LD_SPAN) / 8)) / NLD; };
      auto st_at = [](int x) constexpr { return kStBegin + (x * (((NB - NB1) * DETATTN_ST_SPAN) / 8)) / NLD; };
      static_assert(ld_at(NLD - 1) < NB1 && st_at(NLD - 1) < NB, "RMW slots");
      f32x16 dqAcc[NQB];
#pragma unroll
      for (int m = 0; m < NQB; ++m) dqAcc[m] = f32x16{};
      f32x4 old[NQB][4];
      // dQ tile i in the head's accumulator: uniform byte offset (buffer accesses)
      const int dqtile = (int)(qrow0 * D * 4);
      unsigned char* dqbase = reinterpret_cast<unsigned char*>(a.dqacc + head_off) + dqtile;

      // operand load l (dQ: dS of row block m, K step s; then one per dV/dK MFMA)
      auto loadB = [&](auto lc, Opnd& o) {
        constexpr int l = decltype(lc)::value;
        if constexpr (l < SB_::NL1) {
          constexpr int m = l % C::MQD, s = l / C::MQD;
          static_assert(m == 0, "one dS row block per wave");
          o.lo = lds_tr_asm<16 * s * C::PS>(aS + dsb);
          o.hi = lds_tr_asm<16 * s * C::PS>(aS_hi + dsb);
        } else {
          constexpr int x = l - SB_::NL1, kind = 2 + (x & 1), st = x >> 1;
          constexpr int sq = 2 * (C::MQ - 1) + st / C::ND, n = st % C::ND;
          constexpr int off = (kind == 2 ? C::QB : 0) + 16 * sq * C::PD + 64 * n;
          o.lo = lds_tr_asm<off>(aT);
          o.hi = lds_tr_asm<off + 2 * C::PD>(aT);
        }
      };
      auto mfmaB = [&](auto kc, const u32x4& opr) {
        constexpr int k = decltype(kc)::value;
        const bf16x8 op = as_bf16x8(opr);
        if constexpr (k < NB1) {
          constexpr int l = k / C::DW, n = k % C::DW, m = l % C::MQD, s = l / C::MQD;
          dqAcc[m * C::DW + n] = mfma32(op, kTB[s * C::DW + n], dqAcc[m * C::DW + n]);
        } else {
          constexpr int x = k - NB1, kind = 2 + (x & 1), st = x >> 1;
          constexpr int sq = 2 * (C::MQ - 1) + st / C::ND, n = st % C::ND;
          if constexpr (kind == 2) mfma_agpr(dVacc[n], pB[sq], opr);
          else mfma_agpr(dKacc[n], dsB[sq], opr);
        }
      };
      // element r of block mb, row-major (atomic modes): (uniform tile base) + (32-bit lane offset)
      auto dqp = [&](int mb, int r) -> float* {
        const int m = mb / C::DW, n = mb % C::DW;
        return reinterpret_cast<float*>(dqbase +
                                        (uint32_t)(dqlane_rm + (32 * m + 8 * (r >> 2) + (r & 3)) * D * 4 + 32 * n * 4));
      };
      // register group h of block mb: one 16-byte access per lane, cache scope of the mode
      constexpr int kAux = kScope == __HIP_MEMORY_SCOPE_WORKGROUP ? kBufSc0 : kBufSc1;
      // reads: the first contributor reads a zero-length view (every read out
      // of range returns 0); the resource words are uniform (SGPRs)
      u32x4 ldrsrc;
      {
        const uint64_t p = reinterpret_cast<uint64_t>(a.dqacc + head_off);
        ldrsrc[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
        ldrsrc[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);
        ldrsrc[2] = __builtin_amdgcn_readfirstlane(rk > 0 ? (uint32_t)(a.S * D * 4) : 0u);
        ldrsrc[3] = (uint32_t)kBufferWord3;
      }
      auto dq_load4 = [&](auto xc) -> f32x4 {
        constexpr int x = decltype(xc)::value;
        return buf_load16_asm<(x % 4) * 1024, kAux == kBufSc1>(ldrsrc, dqlane[x / 4], (uint32_t)dqtile);
      };
      auto dq_store4 = [&](int mb, int h, f32x4 v) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), dqrsrc, dqlane[mb] + h * 1024, dqtile, kAux);
      };
      auto acc4 = [&](int mb, int h) -> f32x4 {
        return f32x4{dqAcc[mb][4 * h], dqAcc[mb][4 * h + 1], dqAcc[mb][4 * h + 2], dqAcc[mb][4 * h + 3]};
      };

      // wait for the turn of this workgroup's partial in dQ tile i's order
      auto turn = [&]() {
        if (lane == 0) {
          if (a.delay_seed) {
            const long long until = now_ticks() + (hash3(a.delay_seed, (unsigned)gidx, (unsigned)(t * 4 + w)) & 1023u);
            while (now_ticks() < until) __builtin_amdgcn_s_sleep(2);
          }
          if (seen < turn_val) {
            const long long t0 = now_ticks();
            int spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, kFlagScope) < turn_val) {
              __builtin_amdgcn_s_sleep(1);
              if (((++spins) & 255) == 0) {
                if (now_ticks() - t0 > a.timeout_ticks ||
                    __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                  report_error(a, kErrTimeout);
                  break;
                }
              }
            }
          }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      };
      // RMW modes: read the whole accumulator again (after a late turn) and wait for it
      auto rmw_loads = [&]() {
        if constexpr (DQM == kDqLocalRmw) asm volatile("buffer_inv sc0" ::: "memory");
        static_for<0, NLD>([&](auto xc) {
          constexpr int x = decltype(xc)::value;
          old[x / 4][x % 4] = dq_load4(xc);
        });
        static_for<0, NLD>([&](auto xc) {
          constexpr int x = decltype(xc)::value;
          vm_wait_tied<0>(old[x / 4][x % 4]);
        });
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      };
      // after the dQ MFMAs: wait for the turn if it had not come (RMW: then read
      // the accumulator), or issue the adds themselves (atomic modes)
      auto adds_begin = [&]() {
        if constexpr (kUnordered) {
          // device scope, or (local mode: every add to a dQ tile comes from one XCD) in that XCD's L2
#pragma unroll
          for (int m = 0; m < NQB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              __hip_atomic_fetch_add(dqp(m, r), dqAcc[m][r], __ATOMIC_RELAXED, kScope);
        } else {
          if (!early) {
            turn();
            trace_rec(3, t, gidx);
            if constexpr (kRmw) rmw_loads();
          }
          if constexpr (!kRmw) {  // ordered atomic adds; the first contributor stores
            if (rk == 0) {
#pragma unroll
              for (int m = 0; m < NQB; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  __hip_atomic_store(dqp(m, r), dqAcc[m][r], __ATOMIC_RELAXED, kScope);
            } else {
#pragma unroll
              for (int m = 0; m < NQB; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  __hip_atomic_fetch_add(dqp(m, r), dqAcc[m][r], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
      };
      auto adds_finish = [&]() { trace_rec(4, t, gidx); };

      static_for<0, PF>([&](auto lc) { loadB(lc, ring[decltype(lc)::value]); });
      static_for<0, NB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k == kDecide && !kUnordered) {
          // the flag value is read on every path (also by the first contributor,
          // which does not need it): a load whose result is never used would
          // make the compiler wait for every vector-memory operation before
          // the next write of its register (the next tile's row terms)
          const int seen_u = __builtin_amdgcn_readfirstlane(seen);
          early = rk == 0 || (a.delay_seed == 0 && seen_u >= turn_val);
          // early: the turn has come, the accumulator is read under the dQ MFMAs
          // (local mode drops stale L1 lines first); otherwise it is read after
          // waiting for the turn
          if (early) {
            if constexpr (DQM == kDqLocalRmw) asm volatile("buffer_inv sc0" ::: "memory");
            trace_rec(3, t, gidx);
          }
        }
        if constexpr (kRmw) {
          static_for<0, NLD>([&](auto xc) {
            constexpr int x = decltype(xc)::value;
            // only once the turn has been seen: the accumulator is never read
            // (nor cached) before the previous contributor's adds are visible
            if constexpr (ld_at(x) == k) {
              if (early) old[x / 4][x % 4] = dq_load4(xc);
            }
          });
        }
        if constexpr (k == NB1) {
          DETATTN_FENCE();
          trace_rec(2, t, gidx);
          adds_begin();
          DETATTN_FENCE();
        }
        if constexpr (kRmw) {
          static_for<0, NLD>([&](auto xc) {
            constexpr int x = decltype(xc)::value;
            if constexpr (st_at(x) == k) {
              // read x has landed once at most NLD - 1 later operations are in
              // flight (reads x+1.., writes ..x-1): vector-memory operations
              // complete in issue order. On the late path every read was
              // awaited already.
              vm_wait_tied<NLD - 1>(old[x / 4][x % 4]);
              dq_store4(x / 4, x % 4, old[x / 4][x % 4] + acc4(x / 4, x % 4));
              if constexpr (x == NLD - 1) adds_finish();
            }
          });
        }
        if constexpr (!kRmw && k == kAddLate) {
          adds_finish();
          DETATTN_FENCE();
        }
        // loads that may be issued now (pf loads ahead of this MFMA's own)
        constexpr int l0 = k == 0 ? PF : SB_::issued_by(k - 1, PF) + 1, l1 = SB_::issued_by(k, PF);
        static_for<l0, l1 + 1>([&](auto lc) { loadB(lc, ring[decltype(lc)::value % RING]); });
        constexpr int l = SB_::load_of(k);
        Opnd& o = ring[l % RING];
        // operands are awaited in pairs of loads (l even: l and l + 1)
        if constexpr (SB_::first_use(k) && l % 2 == 0) {
          if constexpr (l + 1 < SB_::NL)
            lgkm_wait2<SB_::insts_after(k, PF) - SB_::ninst(l + 1), false, false>(o, ring[(l + 1) % RING]);
          else
            lgkm_wait<SB_::insts_after(k, PF)>(o.lo, o.hi);
        }
        mfmaB(kc, cat2(o.lo, o.hi));
        DETATTN_FENCE();
      });

      trace_rec(5, t, gidx);
      // The wave publishes its share of the contribution once its adds have
      // landed: early in the next tile's stream A, or at the end of the column.
      // The flag counts wave contributions, so no barrier sits between the
      // adds and the hand-off to the next contributor.
      if constexpr (!kUnordered) {
        const bool withhold = (a.skip_item >= 0 && gidx == a.skip_item && t == 0);
        pend = withhold ? nullptr : flag;
      }
      ++t;
      if (t >= t_end) break;
      cur = nxt;
      b = nb;
      if constexpr (C::NDS == 2) dsb ^= C::SB;
      else lds_barrier();  // the next tile's data is in LDS in every wave's share
    } while (true);  // tiles of the segment

    // ---- end of a column: dK, dV of KV tile j to global ----
    mfma_agpr_drain();
    wait_vm_all();
    if (pend != nullptr) {
      if (lane == 0) __hip_atomic_fetch_add(pend, 1, __ATOMIC_RELAXED, kFlagScope);
      pend = nullptr;
    }
    __syncthreads();
    if constexpr (PAIR && SET == 0) {
      // resident pair: the first column's dK, dV stay in registers until the item ends
      trace_rec(7, t_end, gidx);
      return;
    }
    // every wave's LDS reads and DMA of this column are done: the item's next
    // column's K, V go out now, under the stores below
    if (!PAIR && seg + 1 < sc.segments()) dma_kv(head_off, sc.seg_kv(it, seg + 1));
    {
      float* red = reinterpret_cast<float*>(smem);
      __bf16* sOut = reinterpret_cast<__bf16*>(smem + C::RED_BYTES);
      if constexpr (PAIR) {
        const int j0 = sc.seg_kv(it, 0);
        store_column<C>(dKacc_[0], a.scale, a.dk + head_off + (long long)j0 * BKV * D, red, sOut, wk, wq, lane);
        store_column<C>(dVacc_[0], 1.f, a.dv + head_off + (long long)j0 * BKV * D, red, sOut, wk, wq, lane);
      }
      store_column<C>(dKacc, a.scale, a.dk + head_off + (long long)j * BKV * D, red, sOut, wk, wq, lane);
      store_column<C>(dVacc, 1.f, a.dv + head_off + (long long)j * BKV * D, red, sOut, wk, wq, lane);
    }
    trace_rec(7, t_end, gidx);
    };  // segment body

    if constexpr (PAIR) {
      seg_body(std::integral_constant<int, 0>{}, 0);
      seg_body(std::integral_constant<int, 1>{}, 1);
    } else {
      for (int seg = 0; seg < sc.segments(); ++seg) seg_body(std::integral_constant<int, 0>{}, seg);
    }
  }  // items
}

#undef DETATTN_FENCE

}  // namespace detattn
