/*
 * detattn: deterministic FlashAttention-style attention backward for AMD
 * MI355X (gfx950), with the DASH tile schedules.
 *
 * Operation (all entry points). Softmax attention over one sequence per
 * (batch, head): O = softmax(scale * Q K^T [+ causal mask]) V. The backward
 * produces dQ, dK, dV from Q, K, V, O, dO and the row log-sum-exp. The pages
 * this library follows (DASH: Deterministic Attention Scheduling for
 * High-throughput Reproducible LLM Training; zskr.cn explainer section 2.1 and
 * gist.science summary section 1) describe the tiled backward in which every
 * compute unit produces partial dQ/dK/dV and the dQ partials are reduced
 * globally; a deterministic backward fixes the order of that reduction. The
 * schedules below change only the order in which tiles are visited and dQ
 * partials are added (sections 3.1-3.3 of the explainer; 2.2 of the summary).
 *
 * Conventions shared by every entry point:
 *  - Tensors are contiguous [B, H, S, D], element (b, h, s, d) at
 *    ((b*H + h)*S + s)*D + d. Q, K, V, O, dO, dQ, dK, dV are bf16 (uint16_t
 *    storage, round-to-nearest-even on output). LSE is fp32 [B, H, S], natural
 *    log of sum_j exp(scale * q_i . k_j) over the visible keys.
 *  - Causal mask: key position j is visible from query position i iff j <= i
 *    (one sequence length for queries and keys).
 *  - All tensor and workspace pointers are DEVICE pointers, 16-byte aligned,
 *    owned by the caller. The library never allocates or frees device memory
 *    and keeps no device state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous: they enqueue kernels and return.
 *  - Return value: a detattn_status_t. Argument errors return before anything
 *    is enqueued. No C++ exception crosses this interface.
 *  - Supported now: D in {64, 128}; S a multiple of 64 (and of the chosen KV
 *    tile); B*H*S*D < 2^31 and S*D*4 < 2^31 (one head's fp32 dQ accumulator
 *    is addressed with 32-bit offsets), else DETATTN_ERR_INVALID_ARG. B*H == 0
 *    or S == 0 is a valid empty call.
 */
#ifndef DETATTN_H_
#define DETATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t B, H, S, D;
  float softmax_scale; /* usually 1/sqrt(D) */
} detattn_shape_t;

typedef enum { DETATTN_MASK_FULL = 0, DETATTN_MASK_CAUSAL = 1 } detattn_mask_t;

/*
 * Schedules (order of tile visits and of dQ accumulation):
 *  SERIAL_ASCENDING  each KV tile walks its Q tiles upward; dQ tile i adds the
 *                    KV tiles' partials in ascending order: the FA3
 *                    deterministic baseline (explainer 2.1; summary 1).
 *  DESCENDING_Q      Q tiles from the last down to the first; same dQ order as
 *                    SERIAL_ASCENDING, so dQ is bit-identical to it
 *                    (explainer 3.1; summary 2.2A).
 *  SHIFT             full mask only: the workgroup holding KV tile j starts at
 *                    Q tile j, its own index, and wraps around; dQ order =
 *                    step order (explainer 3.2; summary 2.2B).
 *  SYMMETRIC_SHIFT   causal mask only, even number of KV tiles: KV tiles p and
 *                    n-1-p share a workgroup; dense lower-left rectangle first
 *                    (item p starting at its Q tile p), then the folded
 *                    triangle (explainer 3.3; summary 2.2B): column p upward,
 *                    then column n-1-p downward, each one residue class of
 *                    rows mod r = block_kv / block_q after another.
 *  ATOMIC_NONDET     unordered fp32 atomic adds of the dQ partials: the
 *                    non-deterministic speed reference (explainer 2.1;
 *                    summary 1). dK and dV remain deterministic.
 *  AUTO              the deterministic schedule measured fastest on MI355X
 *                    for the mask (the explainer's future work, section 7,
 *                    chooses the schedule at run time): for causal masks SYMMETRIC_SHIFT,
 *                    except DESCENDING_Q for an odd number of KV tiles and,
 *                    at D = 128, from 128 KV tiles on; for full masks SHIFT.
 *                    The choice depends on the shape only;
 *                    detattn_plan_t.schedule reports it.
 */
typedef enum {
  DETATTN_SERIAL_ASCENDING = 0,
  DETATTN_DESCENDING_Q = 1,
  DETATTN_SHIFT = 2,
  DETATTN_SYMMETRIC_SHIFT = 3,
  DETATTN_ATOMIC_NONDET = 4,
  DETATTN_AUTO = 5
} detattn_schedule_t;

typedef enum {
  DETATTN_OK = 0,
  DETATTN_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad enum, negative size */
  DETATTN_ERR_UNSUPPORTED = 2,   /* valid request this library does not implement */
  DETATTN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  DETATTN_ERR_HIP = 4,           /* a HIP runtime call failed (launch, copy, sync) */
  DETATTN_ERR_DEVICE_TIMEOUT = 5, /* an ordered dQ wait timed out on the device */
  DETATTN_ERR_DEVICE_PLACEMENT = 6, /* no longer returned: XCD-local rings now follow the hardware placement */
  DETATTN_ERR_SCRATCH_LIMIT = 7     /* attn_bwd_deterministic_noalloc: the shape needs more workspace than its
                                       fixed scratch (DETATTN_NOALLOC_SCRATCH_BYTES) holds */
} detattn_status_t;

/* dQ accumulation mechanism for the ordered schedules. */
typedef enum {
  DETATTN_DQ_DEFAULT = 0,
  DETATTN_DQ_ORDERED_RMW = 1,   /* load + add + store of the fp32 accumulator, in rank order */
  DETATTN_DQ_ORDERED_ATOMIC = 2, /* fp32 atomic adds issued in rank order (same order, same bits per run) */
  DETATTN_DQ_XCD_LOCAL_RMW = 3   /* ring schedules whose ring fits one XCD: read-modify-write kept coherent
                                    in that XCD's L2 (never leaves it during the kernel); each workgroup
                                    joins a ring of the XCD the hardware reports it runs on, so the result
                                    does not depend on how workgroups are dispatched to XCDs */
} detattn_dq_mode_t;

/*
 * Optional knobs of attn_bwd_deterministic_ex. Zero-initialise and set what you
 * need; zero always means "library default".
 */
typedef struct {
  int32_t block_q;           /* Q tile rows BQ: 0, 64 or 128 */
  int32_t block_kv;          /* KV tile rows BKV: 0, 64 or 128 (BQ must divide BKV) */
  int32_t grid;              /* persistent workgroups; 0 = one per compute unit x occupancy */
  int32_t xcd_remap;         /* 0 = default (on), 1 = on, 2 = off: keep a ring of workgroups on one XCD */
  int32_t dq_mode;           /* detattn_dq_mode_t */
  uint32_t debug_delay_seed; /* testing: != 0 injects pseudo-random delays before each ordered dQ add */
  uint32_t timeout_us;       /* bound on one ordered wait; 0 = default (4 s) */
  int32_t debug_skip_signal; /* testing: > 0 makes the workgroup of item (debug_skip_signal - 1) never
                                signal its first dQ tile, so its successor times out (forces the
                                failure path; every kernel still exits) */
  void* main_begin_event;    /* optional hipEvent_t recorded on `stream` right before the main kernel */
  void* main_end_event;      /* optional hipEvent_t recorded on `stream` right after the main kernel */
  uint64_t* trace;           /* optional device buffer of grid * trace_records * 2 uint64: per workgroup, records
                                (s_memtime, phase | tile << 8 | item << 32) at the phase boundaries of each
                                tile (detattn_trace_phase_t); unused records stay as the caller left them */
  int32_t trace_records;     /* records per workgroup in `trace` */
  int32_t ring_size;         /* SHIFT / SYMMETRIC_SHIFT: workgroups per ring G, a divisor of the items per head;
                                0 = default, chosen from the shape alone (B*H and the item count) for 8 XCDs
                                of 32 workgroups: the divisor G <= 32 whose rings of one XCD give the shortest
                                makespan (B*H heads, items/G rounds each), larger G on ties; or, when that keeps
                                too little of the chip busy (a prime item count above 32, say), one ring as wide
                                as the item count, spanning XCDs. With power-of-two shapes and at least
                                four heads this is min(items, 32).
                                With G below the item count, workgroup g of a ring takes items g, G+g, ... in
                                rounds, and a dQ tile's order is round-major, step order inside a round
                                (the pages' schedules are the single round G = items per head). G sets the
                                accumulation order: results are bit-identical across calls with the same G.
                                Invalid (UNSUPPORTED) if it does not divide the item count. */
  int32_t dispatch;          /* SERIAL_ASCENDING / DESCENDING_Q / ATOMIC_NONDET: 1 = ticket counter in (head,
                                KV tile) order, 2 = static rings like the shift schedules (ring_size applies;
                                a ring of one XCD keeps the dQ adds in that XCD's L2: read-modify-write for
                                the ordered schedules, fp32 atomic adds for ATOMIC_NONDET), 0 = default:
                                SERIAL_ASCENDING / DESCENDING_Q on rings of one XCD where their estimated
                                makespan beats the ticket counter's (which pays device-scope ordered adds),
                                else on the ticket counter; ATOMIC_NONDET on the ticket counter with
                                device-scope adds (measured faster than adds kept in one XCD's L2). The
                                accumulation order of the ordered schedules, rank = KV tile, is the same
                                in both. Ignored by SHIFT / SYMMETRIC_SHIFT (always rings). */
  int32_t pair_columns;      /* SYMMETRIC_SHIFT: 1 = both columns of a pair item keep their K, V and dK, dV
                                accumulators in registers for the whole item (the pages' alternative to one
                                column at a time; no column switch inside an item, same visits, order and
                                bits); built for D = 64 with 64 x 64 tiles, else UNSUPPORTED. 0 = one
                                column's set at a time (default). */
  int32_t cooperative_launch; /* ring dispatch needs every workgroup of the grid resident at once (a ring's
                                workgroups wait on each other's dQ flags). 0 = default: a plain launch of a
                                grid no larger than the device's resident capacity (compute units x
                                occupancy; a larger explicit `grid` is UNSUPPORTED), which an otherwise idle
                                device runs co-resident; ring calls running at once on other streams of the
                                same device can then hold each other's workgroups back until a bounded wait
                                times out (DETATTN_DEVICE_TIMEOUT, results not deterministic). 1 = HIP's
                                cooperative launch, which guarantees co-residency whatever else runs on the
                                device, at about 15 us of added launch latency per call. Ticket dispatch
                                needs neither (a ticket is only taken by a running workgroup) and always
                                launches plainly. */
  int32_t debug_misplace;    /* testing: 1 = rings of one XCD start from a wrong guess of where each workgroup
                                runs (workgroup w assumes w+1's place), so the placement the hardware reports
                                differs and every workgroup drops its first loads and takes its registered
                                ring; results must not change. No effect elsewhere. */
} detattn_bwd_options_t;

/* Phase ids written into the optional trace (low 8 bits of the second word). */
typedef enum {
  DETATTN_TRACE_TILE_TOP = 0,    /* tile inputs resident, previous flag published */
  DETATTN_TRACE_DS_READY = 1,    /* P, dS computed and dS^T stored in LDS */
  DETATTN_TRACE_DQ_DONE = 2,     /* dQ partial computed (after the dS barrier) */
  DETATTN_TRACE_TURN = 3,        /* the dQ tile's flag reached this tile's rank */
  DETATTN_TRACE_ADDS_ISSUED = 4, /* accumulator adds issued */
  DETATTN_TRACE_TILE_END = 5,    /* dV/dK products issued */
  DETATTN_TRACE_SEG_BEGIN = 6,   /* a KV column starts (K, V staged) */
  DETATTN_TRACE_SEG_END = 7,     /* its dK, dV stored */
  DETATTN_TRACE_WG_START = 8,    /* the workgroup starts (tile field 0) */
  DETATTN_TRACE_REGISTERED = 9   /* XCD-local rings: registration done (tile field = slot, item field = ring) */
} detattn_trace_phase_t;

/* What the library chose for a call (see detattn_bwd_plan). */
typedef struct {
  int32_t block_q, block_kv, n_q, n_kv;
  int32_t items;       /* items over all heads */
  int32_t grid;        /* workgroups launched */
  int32_t ring;        /* workgroups per co-resident ring G (shift schedules), else 0 */
  int32_t rings;       /* rings running at once, else 0 */
  int32_t dq_mode;     /* resolved detattn_dq_mode_t; ATOMIC_NONDET: 0 = device-scope atomic adds,
                          DETATTN_DQ_XCD_LOCAL_RMW = atomic adds in one XCD's L2 (rings of one XCD) */
  int32_t cooperative; /* 1 if launched with HIP's cooperative launch (ring dispatch with cooperative_launch = 1) */
  int32_t schedule;    /* the schedule that runs (AUTO resolved) */
  int32_t pair_columns; /* 1 if the resident-pair form of symmetric shift runs */
} detattn_plan_t;

/*
 * Forward that produces the backward's inputs O and LSE. Not part of the
 * timed backward; deterministic (no cross-workgroup reduction).
 * q, k, v: bf16 [B,H,S,D] in; o: bf16 [B,H,S,D] out; lse: fp32 [B,H,S] out.
 * Requires S % 128 == 0 for now.
 */
int detattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, detattn_shape_t shape,
                detattn_mask_t mask, void* stream);

/* Bytes of device workspace attn_bwd_deterministic needs for `shape`
 * (independent of mask, schedule and options). 0 on invalid shapes. */
size_t detattn_bwd_workspace_bytes(detattn_shape_t shape, detattn_mask_t mask, detattn_schedule_t schedule);

/*
 * Deterministic attention backward (preprocess D = rowsum(dO * O), main kernel,
 * dQ fp32 -> bf16 convert), enqueued on `stream`.
 *  q, k, v, o, dout : bf16 [B,H,S,D] in
 *  lse              : fp32 [B,H,S] in (natural log, as detattn_fwd writes it)
 *  dq, dk, dv       : bf16 [B,H,S,D] out (may not alias inputs)
 *  workspace        : >= detattn_bwd_workspace_bytes(...) bytes, 256-byte aligned;
 *                     overwritten; one workspace per concurrently running call
 * Results are bit-identical across runs for every schedule except
 * ATOMIC_NONDET's dQ; SERIAL_ASCENDING and DESCENDING_Q give identical dQ.
 * Device-side wait timeouts are reported by detattn_device_status.
 */
int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                           detattn_shape_t shape, detattn_mask_t mask, detattn_schedule_t schedule, void* stream);

/* Same as attn_bwd_deterministic with explicit options (NULL = defaults). */
int attn_bwd_deterministic_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, detattn_shape_t shape, detattn_mask_t mask,
                              detattn_schedule_t schedule, const detattn_bwd_options_t* options, void* stream);

/*
 * attn_bwd_deterministic without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is a fixed array in the
 * library's device code, one per GPU, of DETATTN_NOALLOC_SCRATCH_BYTES
 * (136 MiB: every shape with B*H*S*D <= 2^25 at D = 128 or 64, the 8k- and
 * 16k-token workloads included); each GPU the entry point runs on holds it until
 * the process ends. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks the array's
 * device address up (hipGetSymbolAddress) with that device current.
 *  - Arguments, results and bits as attn_bwd_deterministic with default options.
 *  - A shape whose workspace (detattn_bwd_workspace_bytes) exceeds the scratch
 *    returns DETATTN_ERR_SCRATCH_LIMIT before any HIP call.
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last
 *    call's contents (each call clears what must start at zero). Calls that
 *    overlap on one GPU (two streams, two threads) race: serialise them.
 *  - detattn_device_status(NULL, stream) reads the scratch's status word on the
 *    current device.
 */
#define DETATTN_NOALLOC_SCRATCH_BYTES (136ull << 20)
int attn_bwd_deterministic_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, void* dq, void* dk, void* dv, detattn_shape_t shape,
                                   detattn_mask_t mask, detattn_schedule_t schedule, void* stream);

/*
 * Measurement aid for the XCD placement study (not part of the backward): the
 * round-trip latency of a flag passed between workgroups wg_a and wg_b of a
 * small cooperative grid through device-scope atomics, the mechanism of the
 * ordered dQ hand-off (the pages' inter-SM hand-off: nachedeu.com news piece;
 * zskr.cn explainer section 4.2). With round-robin dispatch, workgroups whose
 * indices agree modulo 8 share an XCD.
 *  scratch : device, 256 bytes, 256-byte aligned (overwritten)
 *  result  : device, 5 uint64 (asynchronous; read after synchronising `stream`):
 *            [0] s_memrealtime ticks (100 MHz) and [1] shader cycles over
 *            round_trips - 1 round trips, [2] XCD of wg_a, [3] XCD of wg_b,
 *            [4] 1 if a wait gave up (after 1 s; the kernel always ends)
 *  wg_a, wg_b < 64 and distinct; 2 <= round_trips <= 65536 (all within the 1 s bound).
 * Returns DETATTN_ERR_INVALID_ARG or DETATTN_ERR_HIP before launching on errors.
 */
int detattn_xcd_handoff(int wg_a, int wg_b, int round_trips, void* scratch, uint64_t* result, void* stream);

/* Resolve tiles, grid and rings for a call without launching anything.
 * Needs a HIP device for the compute-unit count unless options->grid > 0. */
int detattn_bwd_plan(detattn_shape_t shape, detattn_mask_t mask, detattn_schedule_t schedule,
                     const detattn_bwd_options_t* options, detattn_plan_t* plan);

/* Synchronise `stream` and read the device status word of `workspace` (NULL:
 * the no-alloc scratch of the current device, once attn_bwd_deterministic_noalloc
 * has run there; before that NULL is DETATTN_ERR_INVALID_ARG): the
 * errors of every call that used it since the status was last read (the word
 * is sticky: a later successful call does not clear it; this read does).
 * DETATTN_OK, DETATTN_ERR_DEVICE_TIMEOUT (an ordered dQ wait, or the start-up
 * registration of XCD-local rings, ran out of time: that call's dQ is not
 * valid), or ERR_HIP. A workspace no call has used yet reads OK. */
int detattn_device_status(void* workspace, void* stream);

/* Static, human-readable name of a status code. */
const char* detattn_status_string(int status);

/*
 * Host-side view of a schedule, the same integer functions the device uses.
 * For item `item` (a KV tile, or a symmetric pair index) of one head with
 * n_q Q tiles and n_kv KV tiles: writes up to `cap` entries of its visit
 * sequence (Q tile, KV tile, rank of that KV tile in the dQ tile's order) and
 * returns the item's length, or -1 on invalid arguments. The entries come from
 * the incremental walk the main kernel takes, checked step by step against the
 * closed-form definitions; -2 reports a disagreement (an internal error).
 */
int detattn_schedule_item(int32_t schedule, int32_t mask, int32_t n_q, int32_t n_kv, int32_t item,
                          int32_t* q_tiles, int32_t* kv_tiles, int32_t* ranks, int32_t cap);

/* The same for a ring of `ring` workgroups (SHIFT and SYMMETRIC_SHIFT only; 0 = one round, as above):
 * the item's visits do not change, its ranks are those of the round-major order that
 * detattn_bwd_options_t.ring_size describes. -1 if `ring` does not divide the item count. */
int detattn_schedule_item_ring(int32_t schedule, int32_t mask, int32_t n_q, int32_t n_kv, int32_t ring,
                               int32_t item, int32_t* q_tiles, int32_t* kv_tiles, int32_t* ranks, int32_t cap);

/* Items per head of a schedule (n_kv, or n_kv/2 for SYMMETRIC_SHIFT); -1 if invalid
 * (including n_q / n_kv not a power of two up to 8). */
int detattn_schedule_items_per_head(int32_t schedule, int32_t mask, int32_t n_q, int32_t n_kv);

#ifdef __cplusplus
}
#endif
#endif /* DETATTN_H_ */
