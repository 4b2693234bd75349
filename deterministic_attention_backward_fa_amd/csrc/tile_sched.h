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
// * shift (full mask): item j starts at Q tile j, its own index, and wraps
//   around; no dQ tile receives two contributions in one step, and the order
//   is the step order (zskr.cn 3.2, gist.science 2.2B). With r = 1 the start is
//   the diagonal block; with r > 1 the items of one step cover n_kv
//   consecutive Q tiles, which move by one per step, so a ring's live dQ and
//   Q/dO tiles stay few (measured 7-8% faster at r = 2 than starting item j
//   at Q tile j*r, whose steps alternate between even and odd tiles).
// * symmetric shift (causal mask): KV tiles p and n_kv-1-p form one item.
//   Phase 1 shifts over the dense lower-left rectangle (Q tiles >= n_q/2, KV
//   tiles < n_kv/2), item p starting at the rectangle's Q tile p, its own
//   index; phase 2 finishes column p upward and then column n_kv-1-p
//   downward, each column one residue class of rows mod r after another (so a
//   step's tiles stay inside one class; each dQ tile's order is that of plain
//   upward and downward rows). Every item holds n_q + r tiles (zskr.cn 3.3,
//   gist.science 2.2B; the fold itself is this library's reading, as the pages
//   give no figure). The order is the step order.
// * atomic (non-deterministic): ascending visits, unordered atomic adds.
//
// Rings of the two shift schedules. The pages' model has one SM per item, all
// in lock step. Here a ring of G workgroups may hold fewer workgroups than a
// head has items: workgroup g then takes items g, G + g, 2G + g, ... in rounds,
// each round right after its previous item. A dQ tile's order is round-major
// and, inside a round, the step order (the lock-step order of that round's G
// items, which are conflict-free as a subset of all items). G = items per head
// is the pages' single round. With G = 32 a ring fits one XCD of MI355X, which
// keeps its dQ hand-offs in that XCD's L2 at any sequence length.
#pragma once

namespace detattn {

// Incremental walk over one segment of an item: the Q tile and rank of each
// step from the previous step's with a few integer operations, so a kernel's
// per-tile bookkeeping needs no division. Sched::walk positions a walk at
// the segment's first step; advance(t) moves it to step t (the next one).
// Every schedule's segment is an arithmetic run of Q tiles with at most one
// wrap-around and at most one jump. A rank is either fixed (the KV tile) or,
// for the shift orders, a function of q, the steps since the segment (or the
// jump) began (divided by r in symmetric shift's phase 2, where a step moves
// r Q tiles between items), and of the Q tile's row block of r tiles:
//   rank = base + min(q, c1) + max(0, q - c2) + max(0, e0 + i / r);
// a fixed rank is base alone (c1 = 0, the other terms vanish).
// With one round (G = items per head) this is q; the other terms count the
// contributions of earlier rounds and the round's own wrap-around.
struct SegWalk {
  static constexpr int kBig = 1 << 28;
  static constexpr int kJumped = -2;  // jump_t once the jump has been taken
  int i;                // Q tile of the current step
  int n;                // steps since the segment (or the jump) began; q = n >> rs
  int di;               // Q tile increment per step (+1 or -1)
  int wrap_at, wrap_to; // a step reaching Q tile wrap_at continues at wrap_to
  int jump_t, jump_i;   // step jump_t continues at Q tile jump_i, n restarts at 0 (kJumped afterwards)
  int rs;               // q = n >> rs (0 where a step moves one Q tile between items, else log2(r))
  int rsi;              // log2(r): Q tile i to its row block of r tiles, i >> rsi
  int rs_jump;          // rs after the jump
  int base, c1, c2, e0; // rank terms; a fixed rank is base with c1 = 0

  __host__ __device__ __forceinline__ int rank_now() const {
    const int q = n >> rs;
    const int lo = q < c1 ? q : c1;
    const int over = q - c2 > 0 ? q - c2 : 0;
    const int late = e0 + (i >> rsi) > 0 ? e0 + (i >> rsi) : 0;
    return base + lo + over + late;
  }

  __host__ __device__ __forceinline__ void advance(int t) {
    i += di;
    if (i == wrap_at) {
      i = wrap_to;
      if (jump_t == kJumped) {  // the next residue class of the run after the jump
        ++wrap_at;
        ++wrap_to;
      }
    }
    ++n;
    if (jump_t == kJumped) n = i - jump_i;
    if (t == jump_t) {
      // the run after the jump (symmetric shift's column above the rectangle)
      // takes one residue class mod r after another, r rows per step: it ends
      // each class where the rectangle begins (the phase-1 wrap target) and
      // continues at the next class, n counting rows from the run's start
      i = jump_i;
      n = 0;
      c2 = kBig;
      e0 = -kBig;
      rs = rs_jump;
      di = 1 << rs_jump;
      wrap_at = wrap_to;
      wrap_to = jump_i + 1;
      jump_t = kJumped;
    }
  }
};

enum Schedule : int { kSerialAscending = 0, kDescendingQ = 1, kShift = 2, kSymmetricShift = 3, kAtomicNondet = 4 };

struct Sched {
  int sch, causal, n_q, n_kv, r;
  int G;  // ring size of the shift schedules (items per round); 0 = items per head (one round)

  __host__ __device__ __forceinline__ int items_per_head() const {
    return sch == kSymmetricShift ? n_kv / 2 : n_kv;
  }
  __host__ __device__ __forceinline__ int ring() const { return G > 0 ? G : items_per_head(); }
  __host__ __device__ __forceinline__ int log2r() const { return r == 1 ? 0 : r == 2 ? 1 : r == 4 ? 2 : 3; }

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

  // KV tile of segment `seg` of item `it`.
  __host__ __device__ __forceinline__ int seg_kv(int it, int seg) const {
    return (sch == kSymmetricShift && seg == 1) ? n_kv - 1 - it : it;
  }

  // The t-th tile (0 <= t < item_len(it)) of item `it`.
  __host__ __device__ __forceinline__ void tile(int it, int t, int& i, int& j) const {
    switch (sch) {
      case kShift:
        j = it;
        i = (it + t) % n_q;
        return;
      case kSymmetricShift: {
        const int half = n_q / 2;
        const int p = it;
        if (t < half) {
          j = p;
          i = half + (p + t) % half;
          return;
        }
        const int t2 = t - half;
        const int top = half - p * r;  // rows p*r .. half-1 of column p
        if (t2 < top) {
          // one residue class mod r after another, L = top / r rows each
          const int L = top / r;
          j = p;
          i = p * r + t2 / L + r * (t2 % L);
        } else {
          // column n_kv-1-p downward, one residue class mod r after another,
          // L = p + 1 rows each
          const int u = t2 - top, L = p + 1;
          j = n_kv - 1 - p;
          i = n_q - r + u / L - r * (u % L);
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
    w.n = 0;
    w.di = 1;
    w.wrap_at = n_q + 1;  // not reached
    w.wrap_to = 0;
    w.jump_t = -1;        // no jump
    w.jump_i = 0;
    w.rs = log2r();
    w.rsi = log2r();
    w.rs_jump = log2r();
    const int Gr = ring();
    const int kG = it - it % Gr, g = it % Gr;  // round start and slot
    w.base = kG;
    w.c1 = Gr - 1 - g;
    w.c2 = SegWalk::kBig;
    w.e0 = -SegWalk::kBig;
    switch (sch) {
      case kShift:
        j = it;
        w.i = it % n_q;
        w.wrap_at = n_q;
        w.wrap_to = 0;
        w.c2 = n_q - 1 - g;
        w.rs = 0;
        break;
      case kSymmetricShift: {
        const int half = n_q / 2;
        const int P = n_kv / 2;
        w.e0 = kG - n_kv + 1;  // bottom-half rows: bottom-branch adds of earlier rounds
        if (seg == 0) {  // phase 1 over rows half.., then column it upward from row it*r
          j = it;
          w.i = half + it % half;
          w.wrap_at = n_q;
          w.wrap_to = half;
          w.jump_t = half;
          w.jump_i = it * r;
          w.c2 = half - 1 - g;
          w.rs = 0;
        } else {         // column n_kv-1-it downward from the last row, after the round's phase 1
          // one residue class mod r after another: each class ends below row
          // j*r and the next starts one row higher at the bottom
          j = n_kv - 1 - it;
          w.i = n_q - r;
          w.di = -r;
          w.wrap_at = j * r - r;
          w.wrap_to = n_q - r + 1;
          w.jump_t = SegWalk::kJumped;  // the wrap moves on to the next class
          w.jump_i = 0;                 // n = i >= 0 (this segment's rank is base + the row term)
          w.base = kG + 2 * Gr - 1 - g;
          w.c1 = 0;
        }
        break;
      }
      case kDescendingQ:
        j = it;
        w.i = n_q - 1;
        w.di = -1;
        w.wrap_at = -2;
        w.base = j;
        w.c1 = 0;
        break;
      default:  // serial ascending, atomic
        j = it;
        w.i = causal ? it * r : 0;
        w.base = j;
        w.c1 = 0;
        break;
    }
    return w;
  }

  // Position of KV tile j in dQ tile i's accumulation order, counted
  // directly: contributions of earlier rounds, then those of the same round
  // at earlier steps.
  __host__ __device__ __forceinline__ int rank(int i, int j) const {
    const int Gr = ring();
    switch (sch) {
      case kShift: {
        const int kG = j - j % Gr, g = j % Gr;
        int t = (i - j) % n_q;
        if (t < 0) t += n_q;
        const int q = t;
        // round items at earlier steps: g' > g before the wrap, g' < g after it
        const int before = q < Gr - 1 - g ? q : Gr - 1 - g;
        const int wrapped = q - (n_q - 1 - g) > 0 ? q - (n_q - 1 - g) : 0;
        return kG + before + wrapped;
      }
      case kSymmetricShift: {
        const int half = n_q / 2, P = n_kv / 2;
        const int u = i / r;
        if (j >= P) {  // bottom branch of item p = n_kv-1-j: after its round's phase 1, larger p first
          const int p = n_kv - 1 - j, kG = p - p % Gr, g = p % Gr;
          const int earlier_bottom = kG - (n_kv - 1 - u) > 0 ? kG - (n_kv - 1 - u) : 0;
          return kG + earlier_bottom + Gr + (Gr - 1 - g);
        }
        const int p = j, kG = p - p % Gr, g = p % Gr;
        if (i >= half) {  // phase 1 on the dense rectangle
          int t = (i - half - p) % half;
          if (t < 0) t += half;
          const int q = t;
          const int earlier_bottom = kG - (n_kv - 1 - u) > 0 ? kG - (n_kv - 1 - u) : 0;
          const int before = q < Gr - 1 - g ? q : Gr - 1 - g;
          const int wrapped = q - (half - 1 - g) > 0 ? q - (half - 1 - g) : 0;
          return kG + earlier_bottom + before + wrapped;
        }
        // top branch: columns p' <= u contribute, later steps for smaller p'
        const int earlier = kG < u + 1 ? kG : u + 1;
        const int last = kG + Gr - 1 < u ? kG + Gr - 1 : u;
        return earlier + last - p;
      }
      default:
        return j;
    }
  }
};

}  // namespace detattn
