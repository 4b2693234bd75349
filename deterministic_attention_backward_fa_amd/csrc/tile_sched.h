// Tile schedules of the deterministic attention backward (integer only,
// evaluated on the host for planning and on the device per tile).
//
// A head's score matrix is cut into n_q query tiles (BQ rows) and n_kv key/value
// tiles (BKV rows), r = BKV / BQ. Tile (i, j) pairs Q tile i with KV tile j.
// An item is the ordered list of tiles one workgroup handles while it keeps
// one KV tile's dK/dV accumulators resident: all work of a KV tile stays on
// one compute unit (DASH; zskr.cn explainer 2.2, gist.science summary 2.1).
// rank(i, j) is KV tile j's position in dQ tile i's accumulation order.
//
// * serial ascending: item j visits its Q tiles upward; dQ order is ascending j
//   (the FA3 deterministic baseline; zskr.cn 2.1, gist.science 1).
// * descending Q: the same loop reversed; the dQ order stays ascending j
//   (zskr.cn 3.1, gist.science 2.2A).
// * shift (full mask): item j starts at Q tile j*r and wraps around; every dQ
//   tile receives one contribution per step, so the order is the step order
//   (zskr.cn 3.2, gist.science 2.2B).
// * symmetric shift (causal mask): KV tiles p and n_kv-1-p form one item.
//   Phase 1 shifts over the dense lower-left rectangle (Q tiles >= n_q/2, KV
//   tiles < n_kv/2); phase 2 finishes column p upward and then column
//   n_kv-1-p downward. Every item holds n_q + r tiles (zskr.cn 3.3,
//   gist.science 2.2B; the fold itself is this library's reading, as the pages
//   give no figure). The order is the step order.
// * atomic (non-deterministic): ascending visits, unordered atomic adds.
#pragma once

namespace detattn {

// Incremental walk over one segment of an item: the Q tile and rank of each
// step from the previous step's with a few integer operations, so a kernel's
// per-tile bookkeeping needs no division. Sched::walk positions a walk at
// the segment's first step; advance(t) moves it to step t (the next one).
// Every schedule's segment is an arithmetic run of Q tiles with at most one
// wrap-around and at most one jump, and its ranks are either the KV tile
// itself or a step counter divided by r (shift orders).
struct SegWalk {
  int i;                // Q tile of the current step
  int rank;             // rank of the current step (when ranked by step)
  int cnt;              // steps taken in the current group of r steps
  int di;               // Q tile increment per step (+1 or -1)
  int wrap_at, wrap_to; // a step reaching Q tile wrap_at continues at wrap_to
  int jump_t, jump_i;   // step jump_t continues at Q tile jump_i, ranks restart at 0
  int r;                // steps per rank (shift orders)
  int fixed_rank;       // the rank of every step, or -1 when ranked by step

  __host__ __device__ __forceinline__ int rank_now() const { return fixed_rank >= 0 ? fixed_rank : rank; }

  __host__ __device__ __forceinline__ void advance(int t) {
    i += di;
    if (i == wrap_at) i = wrap_to;
    ++cnt;
    const bool next_group = cnt == r;
    cnt = next_group ? 0 : cnt;
    rank += next_group ? 1 : 0;
    if (t == jump_t) {
      i = jump_i;
      rank = 0;
      cnt = 0;
    }
  }
};

enum Schedule : int { kSerialAscending = 0, kDescendingQ = 1, kShift = 2, kSymmetricShift = 3, kAtomicNondet = 4 };

struct Sched {
  int sch, causal, n_q, n_kv, r;

  __host__ __device__ __forceinline__ int items_per_head() const {
    return sch == kSymmetricShift ? n_kv / 2 : n_kv;
  }

  __host__ __device__ __forceinline__ int item_len(int it) const {
    switch (sch) {
      case kShift: return n_q;
      case kSymmetricShift: return n_q + r;
      default: return causal ? n_q - it * r : n_q;
    }
  }

  // An item visits one KV tile (one segment) or, for symmetric shift, two KV
  // tiles one after the other (two segments); segments split the item's tile
  // sequence at the column switch.
  __host__ __device__ __forceinline__ int segments() const { return sch == kSymmetricShift ? 2 : 1; }
  __host__ __device__ __forceinline__ int seg_begin(int it, int seg) const {
    return seg == 0 ? 0 : n_q - it * r;  // symmetric: column p holds n_q - p*r tiles
  }
  __host__ __device__ __forceinline__ int seg_end(int it, int seg) const {
    return (sch == kSymmetricShift && seg == 0) ? n_q - it * r : item_len(it);
  }

  // The t-th tile (0 <= t < item_len(it)) of item `it`.
  __host__ __device__ __forceinline__ void tile(int it, int t, int& i, int& j) const {
    switch (sch) {
      case kShift:
        j = it;
        i = (it * r + t) % n_q;
        return;
      case kSymmetricShift: {
        const int half = n_q / 2;
        const int p = it;
        if (t < half) {
          j = p;
          i = half + (p * r + t) % half;
          return;
        }
        const int t2 = t - half;
        const int top = half - p * r;  // rows p*r .. half-1 of column p
        if (t2 < top) {
          j = p;
          i = p * r + t2;
        } else {
          j = n_kv - 1 - p;
          i = n_q - 1 - (t2 - top);
        }
        return;
      }
      case kDescendingQ:
        j = it;
        i = n_q - 1 - t;
        return;
      default:  // serial ascending, atomic
        j = it;
        i = (causal ? it * r : 0) + t;
        return;
    }
  }

  // Walk over segment `seg` of item `it`, at step seg_begin(it, seg); j is the
  // segment's KV tile. Equal, step by step, to tile() and rank().
  __host__ __device__ __forceinline__ SegWalk walk(int it, int seg, int& j) const {
    SegWalk w;
    w.rank = 0;
    w.cnt = 0;
    w.di = 1;
    w.wrap_at = n_q + 1;  // not reached
    w.wrap_to = 0;
    w.jump_t = -1;        // no jump
    w.jump_i = 0;
    w.r = r;
    w.fixed_rank = -1;
    switch (sch) {
      case kShift:
        j = it;
        w.i = (it * r) % n_q;
        w.wrap_at = n_q;
        w.wrap_to = 0;
        break;
      case kSymmetricShift: {
        const int half = n_q / 2;
        if (seg == 0) {  // phase 1 over rows half.., then column it upward from row it*r
          j = it;
          w.i = half + (it * r) % half;
          w.wrap_at = n_q;
          w.wrap_to = half;
          w.jump_t = half;
          w.jump_i = it * r;
        } else {         // column n_kv-1-it downward from the last row
          j = n_kv - 1 - it;
          w.i = n_q - 1;
          w.di = -1;
          w.wrap_at = -2;
          w.fixed_rank = j;
        }
        break;
      }
      case kDescendingQ:
        j = it;
        w.i = n_q - 1;
        w.di = -1;
        w.wrap_at = -2;
        w.fixed_rank = j;
        break;
      default:  // serial ascending, atomic
        j = it;
        w.i = causal ? it * r : 0;
        w.fixed_rank = j;
        break;
    }
    return w;
  }

  // Position of KV tile j in dQ tile i's accumulation order.
  __host__ __device__ __forceinline__ int rank(int i, int j) const {
    switch (sch) {
      case kShift: {
        int d = (i - j * r) % n_q;
        if (d < 0) d += n_q;
        return d / r;
      }
      case kSymmetricShift: {
        const int half = n_q / 2;
        if (j >= n_kv / 2) return j;  // phase-2 bottom branch: after all phase-1 adds, ascending j
        if (i >= half) {              // phase 1 on the dense rectangle
          int d = (i - half - j * r) % half;
          if (d < 0) d += half;
          return d / r;
        }
        return i / r - j;  // phase-2 top branch: later steps belong to smaller p
      }
      default:
        return j;
    }
  }
};

}  // namespace detattn
