// C ABI of libdetattn (declared in include/detattn.h): argument validation,
// tile and grid planning, workspace carving and kernel launches.
#include "detattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "launch.h"
#include "tile_sched.h"

using namespace detattn;

namespace detattn {
void* noalloc_scratch_if_ready();  // noalloc.hip
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sizes the kernels index with 32-bit integers: every element of a call
// (B*H*S*D) and the bytes of one head's fp32 dQ accumulator (S*D*4).
bool shape_ok(const detattn_shape_t& s) {
  if (s.B < 0 || s.H < 0 || s.S < 0 || s.D <= 0) return false;
  const long long n = (long long)s.B * s.H * s.S * s.D;
  return n < (1LL << 31) && (long long)s.S * s.D * 4 < (1LL << 31);
}

bool is_empty(const detattn_shape_t& s) { return s.B == 0 || s.H == 0 || s.S == 0; }

// Library tile choice per head dimension and length: the KV tile (BKV rows,
// owned by one workgroup) and the Q tile (BQ rows, one sweep step), the
// fastest measured on MI355X. At D = 128 the 128-row KV tile wins at every
// length, 16k included, where the pages advise a smaller one for H800's
// registers (explainer section 5.3): gfx950 keeps K, V and dK, dV of a
// 128-row tile in its 512 registers per lane.
void default_tiles(int D, int S, int& bq, int& bkv) {
  if (D == 64) {
    if (S % 128 == 0 && S >= 512) {
      bq = 128;
      bkv = 128;
    } else {
      bq = 64;
      bkv = 64;
    }
  } else {
    bq = 64;
    bkv = S % 128 == 0 ? 128 : 64;
  }
}

bool tiles_built(int D, int bq, int bkv) {
  if (D == 64) return (bq == 64 && bkv == 64) || (bq == 128 && bkv == 128) || (bq == 64 && bkv == 128);
  if (D == 128) return (bq == 64 && bkv == 128) || (bq == 64 && bkv == 64);
  return false;
}

// MI355X: 256 compute units in 8 XCDs, one main-kernel workgroup each.
constexpr int kXcds = 8;
constexpr int kXcdSlots = 32;
// Measured cost of dQ hand-offs that leave one XCD's L2, relative to rings of
// one XCD: one ring per head spanning XCDs ran 2.0-2.5x slower (16k tokens),
// the ticket counter with device-scope ordered adds 1.6-1.9x slower.
constexpr double kCrossRingCost = 2.0;
constexpr double kTicketCost = 1.8;

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Makespan, in item times, of BH heads of ip items each on rings of G
// workgroups confined to one XCD, with `slots_per_xcd` workgroups per XCD: each
// XCD runs floor(slots / G) rings (no more than its share of the heads needs),
// and a ring takes its heads one after the other, ip / G rounds each.
double local_ring_cost(long long BH, int ip, int G, int slots_per_xcd) {
  const long long per_xcd = slots_per_xcd / G;
  if (per_xcd == 0 || ip % G != 0) return 1e300;
  const long long rings = kXcds * std::min(per_xcd, ceil_div(BH, kXcds));
  return (double)ceil_div(BH, rings) * (ip / G);
}

// The same for one ring per head as wide as its item count (the pages' single
// round), spanning XCDs, with `slots` workgroups in all.
double cross_ring_cost(long long BH, int ip, int slots) {
  const long long rings = std::min<long long>(slots / ip, BH);
  if (rings == 0) return 1e300;
  return (double)ceil_div(BH, rings) * kCrossRingCost;
}

// Default ring size G of the shift schedules: the divisor of the item count
// up to one XCD's 32 workgroups (or, when none keeps enough of the chip busy,
// the whole item count on a ring spanning XCDs) with the shortest makespan
// above, larger G on ties (measured faster at equal makespan). It is chosen for
// MI355X's nominal 8 x 32 workgroups and depends on the shape only: G sets the
// accumulation order, so every bit of dQ is independent of the grid.
int default_ring(long long BH, int ip) {
  int best = 1;
  double best_cost = 1e301;
  for (int g = std::min(ip, kXcdSlots); g >= 1; --g) {
    const double c = local_ring_cost(BH, ip, g, kXcdSlots);
    if (c < best_cost) {
      best = g;
      best_cost = c;
    }
  }
  if (ip > kXcdSlots && cross_ring_cost(BH, ip, kXcds * kXcdSlots) < best_cost) best = ip;
  return best;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

struct Plan {
  detattn_plan_t pub;
  int causal, sch, dqm_internal, xcd;
  Sched sc;
  long long timeout_ticks;
};

int make_plan(const detattn_shape_t& s, detattn_mask_t mask, detattn_schedule_t sch, const detattn_bwd_options_t* opt,
              Plan& P) {
  if (!shape_ok(s) || is_empty(s)) return DETATTN_ERR_INVALID_ARG;
  if (mask != DETATTN_MASK_FULL && mask != DETATTN_MASK_CAUSAL) return DETATTN_ERR_INVALID_ARG;
  if ((int)sch < 0 || (int)sch > 5) return DETATTN_ERR_INVALID_ARG;
  if (s.D != 64 && s.D != 128) return DETATTN_ERR_UNSUPPORTED;
  detattn_bwd_options_t o;
  std::memset(&o, 0, sizeof(o));
  if (opt) o = *opt;
  if (o.block_q < 0 || o.block_kv < 0 || o.grid < 0 || o.xcd_remap < 0 || o.xcd_remap > 2 || o.dq_mode < 0 ||
      o.dq_mode > 3 || o.ring_size < 0 || o.dispatch < 0 || o.dispatch > 2 || o.pair_columns < 0 ||
      o.pair_columns > 1 || o.cooperative_launch < 0 || o.cooperative_launch > 1 || o.debug_misplace < 0 ||
      o.debug_misplace > 1)
    return DETATTN_ERR_INVALID_ARG;
  int bq, bkv;
  default_tiles(s.D, s.S, bq, bkv);
  if (o.block_q) bq = o.block_q;
  if (o.block_kv) bkv = o.block_kv;
  if (!tiles_built(s.D, bq, bkv)) return DETATTN_ERR_UNSUPPORTED;
  if (s.S % bq != 0 || s.S % bkv != 0) return DETATTN_ERR_UNSUPPORTED;
  const int causal = mask == DETATTN_MASK_CAUSAL;
  const int n_q = s.S / bq, n_kv = s.S / bkv, r = bkv / bq;
  // AUTO: the fastest deterministic schedule measured on MI355X. Full:
  // shift. Causal: symmetric shift, except descending for an odd KV-tile
  // count and, at D = 128, from 128 KV tiles on (several rounds of items per
  // ring, where descending's snake order measured 0.4-2.5% ahead; at 64 KV
  // tiles symmetric shift measured ahead).
  if (sch == DETATTN_AUTO)
    sch = !causal                          ? DETATTN_SHIFT
          : n_kv % 2 != 0                  ? DETATTN_DESCENDING_Q
          : (s.D == 128 && n_kv >= 128)    ? DETATTN_DESCENDING_Q
                                           : DETATTN_SYMMETRIC_SHIFT;
  if (sch == DETATTN_SHIFT && causal) return DETATTN_ERR_UNSUPPORTED;
  if (sch == DETATTN_SYMMETRIC_SHIFT && (!causal || n_kv % 2 != 0)) return DETATTN_ERR_UNSUPPORTED;

  // The kernel instance depends on the dQ mode, which depends on the ring
  // placement below; occupancy (LDS-bound) is the same for every mode.
  const MainInfo info0 = main_info(s.D, bq, bkv, causal, kDqOrderedRmw, false);
  if (!info0.func) return DETATTN_ERR_UNSUPPORTED;

  Sched sc{(int)sch, causal, n_q, n_kv, r, 0};
  const int ip = sc.items_per_head();
  const long long BH = (long long)s.B * s.H;
  const long long items = BH * ip;
  int capacity = 0;  // co-resident workgroups
  int cus = 0;
  if (o.grid == 0) {
    cus = device_cus();
    if (cus <= 0 || info0.occupancy <= 0) return DETATTN_ERR_HIP;
    capacity = cus * info0.occupancy;
  }
  int grid = o.grid ? o.grid : capacity;
  int ring = 0, rings = 0;
  int xcd = o.xcd_remap != 2;
  // Shift schedules always run on rings. Serial and descending run on rings
  // too where a ring fits one XCD (their ordered adds then stay in that XCD's
  // L2), else on the ticket counter; the order (rank = KV tile) is the same.
  // The atomic reference stays on the ticket counter with device-scope adds
  // unless asked: its adds confined to one XCD's L2 measured slower.
  bool ring_sched = sch == DETATTN_SHIFT || sch == DETATTN_SYMMETRIC_SHIFT;
  int ring_pref = o.ring_size;
  if (sch == DETATTN_SERIAL_ASCENDING || sch == DETATTN_DESCENDING_Q || sch == DETATTN_ATOMIC_NONDET) {
    // rank = KV tile whatever the dispatch: the ring size may follow the grid
    const bool local_fits = xcd && grid % kXcds == 0 && grid >= kXcds && grid <= (int)WsLayout::kMaxXcdGrid;
    if (!ring_pref) {
      ring_pref = 1;
      double best = 1e301;
      const int slots = local_fits ? grid / kXcds : 0;
      for (int g = std::min(ip, std::max(slots, 1)); g >= 1; --g) {
        const double c = local_fits ? local_ring_cost(BH, ip, g, slots) : 1e300;
        if (c < best) {
          best = c;
          ring_pref = g;
        }
      }
      if (o.dispatch == 0 && sch != DETATTN_ATOMIC_NONDET)
        ring_sched = local_fits && best <= (double)ceil_div(items, grid) * kTicketCost;
    } else if (o.dispatch == 0 && sch != DETATTN_ATOMIC_NONDET) {
      ring_sched = local_fits && ring_pref <= grid / kXcds && ip % ring_pref == 0;
    }
    if (o.dispatch == 2) ring_sched = true;
  } else if (!ring_pref) {
    ring_pref = default_ring(BH, ip);
  }
  if (ring_sched) {
    // Every ring (G workgroups sharing one head's items) must be co-resident.
    // With rings of one XCD, each XCD runs `rings / 8` of them, so their dQ
    // hand-offs stay inside that XCD's L2: in the XCD-local modes workgroups
    // join rings by the XCD the hardware reports, otherwise workgroup w is
    // taken to run on XCD w % 8 (a placement only performance depends on).
    sc.G = ring_pref;
    if (ip % sc.G != 0) return DETATTN_ERR_UNSUPPORTED;
    ring = sc.G;
    if (grid < ring) return DETATTN_ERR_UNSUPPORTED;
    if (xcd && grid % 8 == 0 && ring <= grid / 8 && grid <= (int)WsLayout::kMaxXcdGrid) {
      long long per_xcd = (grid / 8) / ring;
      const long long need = (BH + 7) / 8;
      if (per_xcd > need) per_xcd = need;
      rings = (int)(8 * per_xcd);
    } else {
      xcd = 0;
      rings = grid / ring;
      if ((long long)rings > BH) rings = (int)BH;
    }
    grid = rings * ring;
  } else {
    xcd = 0;
    if ((long long)grid > items) grid = (int)items;
  }

  // dQ accumulation mode
  // (ATOMIC_NONDET: unordered atomic adds, in one XCD's L2 when its rings sit on one XCD)
  int dqm = ring_sched && xcd ? kDqUnorderedLocal : kDqUnordered;
  int pub_dqm = dqm == kDqUnorderedLocal ? DETATTN_DQ_XCD_LOCAL_RMW : 0;
  if (sch != DETATTN_ATOMIC_NONDET) {
    const bool local_ok = ring_sched && xcd;
    pub_dqm = o.dq_mode;
    if (pub_dqm == DETATTN_DQ_DEFAULT) pub_dqm = local_ok ? DETATTN_DQ_XCD_LOCAL_RMW : DETATTN_DQ_ORDERED_ATOMIC;
    if (pub_dqm == DETATTN_DQ_XCD_LOCAL_RMW && !local_ok) return DETATTN_ERR_UNSUPPORTED;
    dqm = pub_dqm == DETATTN_DQ_ORDERED_ATOMIC ? kDqOrderedAtomic
          : pub_dqm == DETATTN_DQ_XCD_LOCAL_RMW ? kDqLocalRmw
                                                 : kDqOrderedRmw;
  }
  // the resident pair is symmetric shift's; it has no traced instance
  if (o.pair_columns && (sch != DETATTN_SYMMETRIC_SHIFT || o.trace)) return DETATTN_ERR_UNSUPPORTED;
  const MainInfo info = main_info(s.D, bq, bkv, causal, dqm, false, o.pair_columns != 0);
  if (!info.func) return DETATTN_ERR_UNSUPPORTED;
  P.pub.block_q = bq;
  P.pub.block_kv = bkv;
  P.pub.n_q = n_q;
  P.pub.n_kv = n_kv;
  P.pub.items = (int32_t)items;
  P.pub.grid = grid;
  P.pub.ring = ring;
  P.pub.rings = rings;
  P.pub.dq_mode = pub_dqm;
  P.pub.cooperative = ring_sched && o.cooperative_launch == 1 ? 1 : 0;
  P.pub.schedule = (int32_t)sch;
  P.pub.pair_columns = o.pair_columns;
  P.causal = causal;
  P.sch = (int)sch;
  P.sc = sc;
  P.dqm_internal = dqm;
  P.xcd = xcd;
  const long long us = o.timeout_us ? (long long)o.timeout_us : 4000000LL;
  P.timeout_ticks = us * 100;  // s_memrealtime runs at 100 MHz
  return DETATTN_OK;
}

}  // namespace

extern "C" {

const char* detattn_status_string(int status) {
  switch (status) {
    case DETATTN_OK: return "ok";
    case DETATTN_ERR_INVALID_ARG: return "invalid argument";
    case DETATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case DETATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case DETATTN_ERR_HIP: return "HIP runtime error";
    case DETATTN_ERR_DEVICE_TIMEOUT: return "ordered dQ wait timed out on the device";
    case DETATTN_ERR_DEVICE_PLACEMENT: return "a workgroup ran on an unexpected XCD (no longer reported)";
    case DETATTN_ERR_SCRATCH_LIMIT: return "shape needs more workspace than the no-alloc scratch holds";
    default: return "unknown status";
  }
}

size_t detattn_bwd_workspace_bytes(detattn_shape_t s, detattn_mask_t mask, detattn_schedule_t schedule) {
  (void)mask;
  (void)schedule;
  if (!shape_ok(s)) return 0;
  WsLayout L((long long)s.B * s.H, s.S, s.D);
  return L.total;
}

int detattn_bwd_plan(detattn_shape_t shape, detattn_mask_t mask, detattn_schedule_t schedule,
                     const detattn_bwd_options_t* options, detattn_plan_t* plan) {
  if (!plan) return DETATTN_ERR_INVALID_ARG;
  Plan P;
  const int st = make_plan(shape, mask, schedule, options, P);
  if (st == DETATTN_OK) *plan = P.pub;
  return st;
}

int attn_bwd_deterministic_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, detattn_shape_t s, detattn_mask_t mask,
                              detattn_schedule_t schedule, const detattn_bwd_options_t* options, void* stream) {
  if (!shape_ok(s)) return DETATTN_ERR_INVALID_ARG;
  if (mask != DETATTN_MASK_FULL && mask != DETATTN_MASK_CAUSAL) return DETATTN_ERR_INVALID_ARG;
  if ((int)schedule < 0 || (int)schedule > 5) return DETATTN_ERR_INVALID_ARG;
  if (is_empty(s)) return DETATTN_OK;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return DETATTN_ERR_INVALID_ARG;
  if (options && options->trace &&
      (options->trace_records <= 0 || (reinterpret_cast<uintptr_t>(options->trace) & 7u) != 0))
    return DETATTN_ERR_INVALID_ARG;
  Plan P;
  const int st = make_plan(s, mask, schedule, options, P);
  if (st != DETATTN_OK) return st;
  if (P.pub.ring > 0 && !P.pub.cooperative) {
    // a plain launch of ring dispatch: the whole grid must fit the device at once
    const MainInfo mi = main_info(s.D, P.pub.block_q, P.pub.block_kv, P.causal, P.dqm_internal,
                                  options && options->trace, P.pub.pair_columns != 0);
    const int cus = device_cus();
    if (cus <= 0 || mi.occupancy <= 0) return DETATTN_ERR_HIP;
    if (P.pub.grid > cus * mi.occupancy) return DETATTN_ERR_UNSUPPORTED;
  }
  const long long BH = (long long)s.B * s.H;
  WsLayout L(BH, s.S, s.D);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < L.total)
    return DETATTN_ERR_WORKSPACE;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  unsigned* header = reinterpret_cast<unsigned*>(ws);
  int* flags = reinterpret_cast<int*>(ws + L.flags_off);
  float* ndelta = reinterpret_cast<float*>(ws + L.ndelta_off);
  float* nlse = reinterpret_cast<float*>(ws + L.nlse_off);
  float* dqacc = reinterpret_cast<float*>(ws + L.dqacc_off);
  hipStream_t st_ = static_cast<hipStream_t>(stream);
  const long long rows = BH * s.S;
  const long long elems = rows * s.D;
  const bool unordered = P.dqm_internal == kDqUnordered || P.dqm_internal == kDqUnorderedLocal;

  // the XCD registration table is cleared for the rings of one XCD that register
  const int n_tab = (P.pub.ring > 0 && P.xcd) ? P.pub.grid : 0;
  hipError_t e = launch_pre(s.D, static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), lse,
                            nlse, ndelta, rows, flags, BH * P.pub.n_q, header,
                            reinterpret_cast<unsigned*>(ws + L.xcdtab_off), n_tab, unordered ? dqacc : nullptr,
                            elems, st_);
  if (e != hipSuccess) return DETATTN_ERR_HIP;
  MainLaunch M;
  std::memset(&M, 0, sizeof(M));
  BwdArgs& a = M.args;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.dout = static_cast<const __bf16*>(dout);
  a.nlse = nlse;
  a.ndelta = ndelta;
  a.dqacc = dqacc;
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.flags = flags;
  a.ticket = header + kHdrTicket;
  a.err = header + kHdrAbort;
  a.sticky = header + kHdrSticky;
  a.xcd_tab = reinterpret_cast<unsigned*>(ws + L.xcdtab_off);
  a.BH = (int)BH;
  a.S = s.S;
  a.scale = s.softmax_scale;
  a.sc = P.sc;
  a.ticket_mode = P.pub.ring == 0;
  a.ring = P.pub.ring;
  a.rings = P.pub.rings;
  // Descending items shrink with j under a causal mask: snake order balances a
  // workgroup's rounds (ranks do not depend on the workgroup), measured 14-23%
  // faster. Serial measured slower with it: there a dQ tile's ascending chain
  // waits for the longest items first, so it keeps the plain order.
  a.snake = P.causal && P.sch == kDescendingQ;
  a.xcd_remap = P.xcd;
  a.timeout_ticks = P.timeout_ticks;
  a.delay_seed = options ? options->debug_delay_seed : 0u;
  a.skip_item = (options && options->debug_skip_signal > 0) ? options->debug_skip_signal - 1 : -1;
  a.misplace = options ? options->debug_misplace : 0;
  if (options && options->trace) {
    a.trace = reinterpret_cast<unsigned long long*>(options->trace);
    a.trace_records = options->trace_records;
  }
  M.D = s.D;
  M.BQ = P.pub.block_q;
  M.BKV = P.pub.block_kv;
  M.causal = P.causal;
  M.dq_mode = P.dqm_internal;
  M.grid = P.pub.grid;
  M.cooperative = P.pub.cooperative;
  M.pair = P.pub.pair_columns;
  if (options && options->main_begin_event &&
      hipEventRecord(static_cast<hipEvent_t>(options->main_begin_event), st_) != hipSuccess)
    return DETATTN_ERR_HIP;
  e = launch_main(M, st_);
  if (e == hipSuccess && options && options->main_end_event)
    e = hipEventRecord(static_cast<hipEvent_t>(options->main_end_event), st_);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return e == hipErrorCooperativeLaunchTooLarge ? DETATTN_ERR_UNSUPPORTED : DETATTN_ERR_HIP;
  }
  const bool fragment_order = P.dqm_internal == kDqOrderedRmw || P.dqm_internal == kDqLocalRmw;
  e = launch_convert(s.D, dqacc, static_cast<__bf16*>(dq), rows, s.softmax_scale, fragment_order, st_);
  return e == hipSuccess ? DETATTN_OK : DETATTN_ERR_HIP;
}

int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                           detattn_shape_t shape, detattn_mask_t mask, detattn_schedule_t schedule, void* stream) {
  return attn_bwd_deterministic_ex(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, shape, mask,
                                   schedule, nullptr, stream);
}

int detattn_device_status(void* workspace, void* stream) {
  if (!workspace) workspace = noalloc_scratch_if_ready();
  if (!workspace) return DETATTN_ERR_INVALID_ARG;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return DETATTN_ERR_HIP;
  // the sticky word and its tag (words kHdrSticky .. kHdrTag + 1)
  unsigned w[4] = {0, 0, 0, 0};
  unsigned* header = static_cast<unsigned*>(workspace);
  if (hipMemcpy(w, header + kHdrSticky, sizeof(w), hipMemcpyDeviceToHost) != hipSuccess) return DETATTN_ERR_HIP;
  unsigned long long tag;
  std::memcpy(&tag, w + (kHdrTag - kHdrSticky), sizeof(tag));
  if (tag != kStickyTag || w[0] == kErrNone) return DETATTN_OK;  // no call yet, or no error since the last read
  const unsigned zero = 0;
  if (hipMemcpy(header + kHdrSticky, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return DETATTN_ERR_HIP;
  return DETATTN_ERR_DEVICE_TIMEOUT;
}

int detattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, detattn_shape_t s,
                detattn_mask_t mask, void* stream) {
  if (!shape_ok(s)) return DETATTN_ERR_INVALID_ARG;
  if (mask != DETATTN_MASK_FULL && mask != DETATTN_MASK_CAUSAL) return DETATTN_ERR_INVALID_ARG;
  if (is_empty(s)) return DETATTN_OK;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return DETATTN_ERR_INVALID_ARG;
  if (s.D != 64 && s.D != 128) return DETATTN_ERR_UNSUPPORTED;
  if (s.S % 128 != 0) return DETATTN_ERR_UNSUPPORTED;
  hipError_t e = launch_fwd(s.D, mask == DETATTN_MASK_CAUSAL, static_cast<const __bf16*>(q),
                            static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse,
                            s.B * s.H, s.S, s.softmax_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DETATTN_OK : DETATTN_ERR_HIP;
}

int detattn_schedule_items_per_head(int32_t schedule, int32_t mask, int32_t n_q, int32_t n_kv) {
  if (schedule < 0 || schedule > 4 || (mask != 0 && mask != 1) || n_q <= 0 || n_kv <= 0 || n_q % n_kv != 0)
    return -1;
  const int r = n_q / n_kv;
  if (r != 1 && r != 2 && r != 4 && r != 8) return -1;  // tiles are powers of two
  if (schedule == kShift && mask != 0) return -1;
  if (schedule == kSymmetricShift && (mask != 1 || n_kv % 2 != 0)) return -1;
  const Sched sc{schedule, mask, n_q, n_kv, n_q / n_kv, 0};
  return sc.items_per_head();
}

int detattn_schedule_item_ring(int32_t schedule, int32_t mask, int32_t n_q, int32_t n_kv, int32_t ring,
                               int32_t item, int32_t* q_tiles, int32_t* kv_tiles, int32_t* ranks, int32_t cap) {
  const int ip = detattn_schedule_items_per_head(schedule, mask, n_q, n_kv);
  if (ip < 0 || item < 0 || item >= ip || cap < 0 || ring < 0) return -1;
  const bool ring_sched = schedule == kShift || schedule == kSymmetricShift;
  if (ring > 0 && (!ring_sched || ip % ring != 0)) return -1;
  const Sched sc{schedule, mask, n_q, n_kv, n_q / n_kv, ring};
  const int len = sc.item_len(item);
  // the incremental walk the device takes, checked step by step against the
  // closed forms tile() and rank()
  for (int seg = 0; seg < sc.segments(); ++seg) {
    int j;
    SegWalk wk = sc.walk(item, seg, j);
    for (int t = sc.seg_begin(item, seg); t < sc.seg_end(item, seg); ++t) {
      if (t > sc.seg_begin(item, seg)) wk.advance(t);
      int ci, cj;
      sc.tile(item, t, ci, cj);
      if (ci != wk.i || cj != j || (schedule != kAtomicNondet && sc.rank(ci, cj) != wk.rank_now())) return -2;
      if (t < cap) {
        if (q_tiles) q_tiles[t] = wk.i;
        if (kv_tiles) kv_tiles[t] = j;
        if (ranks) ranks[t] = schedule == kAtomicNondet ? -1 : wk.rank_now();
      }
    }
  }
  return len;
}

int detattn_schedule_item(int32_t schedule, int32_t mask, int32_t n_q, int32_t n_kv, int32_t item, int32_t* q_tiles,
                          int32_t* kv_tiles, int32_t* ranks, int32_t cap) {
  return detattn_schedule_item_ring(schedule, mask, n_q, n_kv, 0, item, q_tiles, kv_tiles, ranks, cap);
}

}  // extern "C"
