"""Tile orders of the pages' schedules, written from their prose.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). This module is the oracle's
own statement of the schedules; the HIP library has its own, independent one,
and the tests compare the two.

Vocabulary
----------
A head's attention matrix is cut into n_q query (Q/dQ) tiles of BQ rows and
n_kv key/value (KV) tiles of BKV rows, r = BKV / BQ (an integer >= 1), so
n_q = r * n_kv. Tile (i, j) pairs Q tile i with KV tile j.

An *item* is the ordered list of tiles one workgroup processes for one KV tile
(or one pair of KV tiles), keeping that KV tile's dK/dV accumulators on chip:
all work of one KV tile runs contiguously on one SM (DASH, zskr.cn explainer
section 2.2; gist.science summary section 2.1, "Vincoli").

The *accumulation order* of dQ tile i is the order in which the KV tiles' dQ
partials are added into it. ``rank(i, j)`` is the position of KV tile j in it.

Causal visibility: key position kv is visible from query position q iff
kv <= q (same sequence for both), so tile (i, j) has at least one visible pair
iff (i + 1) * BQ - 1 >= j * BKV, i.e. i >= j * r.
"""
from typing import Dict, List, Tuple

SCHEDULES = ("serial_ascending", "descending_q", "shift", "symmetric_shift", "atomic_nondet")
MASKS = ("full", "causal")

Tile = Tuple[int, int]


def tile_visible(i: int, j: int, r: int, causal: bool) -> bool:
    return (not causal) or i >= j * r


def column_rows(j: int, n_q: int, r: int, causal: bool) -> List[int]:
    """Q tiles that interact with KV tile j, ascending."""
    return [i for i in range(n_q) if tile_visible(i, j, r, causal)]


def valid(schedule: str, mask: str, n_q: int, n_kv: int) -> bool:
    """Shift is defined for full masks and symmetric shift for causal masks
    (zskr.cn explainer sections 3.2 and 3.3; gist.science summary section 2.2B);
    symmetric shift pairs KV tiles i and N-1-i, so it needs an even count."""
    if schedule == "shift":
        return mask == "full"
    if schedule == "symmetric_shift":
        return mask == "causal" and n_kv % 2 == 0
    return schedule in SCHEDULES


def items(schedule: str, mask: str, n_q: int, n_kv: int) -> List[List[Tile]]:
    """Per-head items, each the list of tiles in visit order.

    serial_ascending: KV tile j walks its Q tiles upward, the FA3 deterministic
        baseline (zskr.cn section 2.1; gist.science section 1).
    descending_q: the same loop reversed, Q tiles from the last down to the
        first (zskr.cn section 3.1; gist.science section 2.2A).
    atomic_nondet: ascending visits; order of dQ adds not fixed.
    shift: the SM holding KV tile j starts at its own index and wraps around,
        visiting j, j+1, ..., N-1, 0, ..., j-1 (zskr.cn section 3.2; gist.science
        section 2.2B). The start is Q tile j, the SM's own index, for any r (with
        r = 1 that is the diagonal block).
    symmetric_shift: KV tiles p and n_kv-1-p form one item. Phase 1 is a shift
        over the dense lower-left rectangle (Q tiles in the bottom half, KV tiles
        in the left half), item p starting at the rectangle's Q tile p, its own
        index; phase 2 finishes column p above the rectangle, then column
        n_kv-1-p, descending (zskr.cn section 3.3; gist.science section 2.2B).
        Column p's rows above the rectangle start at row p*r; they are taken
        ascending one residue class mod r after another (rows p*r, p*r + r, ...,
        then p*r + 1, p*r + 1 + r, ...), and column n_kv-1-p's rows descending
        the same way (rows n_q - r, n_q - 2r, ..., then n_q - r + 1, ...), so
        the items of one step stay inside one class of rows. Each dQ tile
        receives its partials in the same order as with plain ascending and
        descending rows (larger p first), so only the visit order inside an
        item differs. The pages give no figure of the fold; this is the plainest
        construction with one accumulator set live at a time.
    """
    causal = mask == "causal"
    r = n_q // n_kv
    assert r * n_kv == n_q and r >= 1, "BQ must divide BKV"
    if not valid(schedule, mask, n_q, n_kv):
        raise ValueError(f"{schedule} is not defined for mask {mask} with n_kv={n_kv}")
    out: List[List[Tile]] = []
    if schedule in ("serial_ascending", "atomic_nondet"):
        for j in range(n_kv):
            out.append([(i, j) for i in column_rows(j, n_q, r, causal)])
    elif schedule == "descending_q":
        for j in range(n_kv):
            out.append([(i, j) for i in reversed(column_rows(j, n_q, r, causal))])
    elif schedule == "shift":
        for j in range(n_kv):
            out.append([((j + t) % n_q, j) for t in range(n_q)])
    elif schedule == "symmetric_shift":
        half = n_q // 2
        for p in range(n_kv // 2):
            seq = [(half + (p + t) % half, p) for t in range(half)]
            # column p above the rectangle, rows p*r .. half-1, one residue
            # class mod r after another (r = 1: simply ascending)
            seq += [(i, p) for k in range(r) for i in range(p * r + k, half, r)]
            c = n_kv - 1 - p
            # column c downward from the last row, likewise one residue class
            # mod r after another (rows n_q-r, n_q-2r, ..., then n_q-r+1, ...)
            seq += [(i, c) for k in range(r) for i in range(n_q - r + k, c * r - 1, -r)]
            out.append(seq)
    return out


def accumulation_order(schedule: str, mask: str, n_q: int, n_kv: int, ring: int = 0) -> Dict[int, List[int]]:
    """dQ tile i -> KV tiles in the order their partials are added.

    serial_ascending and descending_q both keep FA3's ascending KV order; the
    descending heuristic only reverses the loop that visits Q tiles (zskr.cn
    section 3.1). For shift and symmetric shift, every item advances one tile
    per step in lock step and the contributions to a dQ tile are added in step
    order, which the pages describe as forming a natural dependency chain with
    no conflicts (zskr.cn section 3.2; gist.science section 2.2B).

    ``ring`` (shift schedules only): the number of workgroups that share a
    head's items when there are fewer of them than items. The pages' model has
    one SM per item; this reading extends it: workgroup g takes items g,
    ring + g, 2 ring + g, ... one round after another, the items of one round
    run in lock step, and a dQ tile takes its partials round by round, in step
    order inside a round. 0 (or the item count) is the pages' single round.
    """
    if schedule == "atomic_nondet":
        raise ValueError("atomic_nondet has no fixed accumulation order")
    causal = mask == "causal"
    r = n_q // n_kv
    order: Dict[int, List[int]] = {}
    if schedule in ("serial_ascending", "descending_q"):
        for i in range(n_q):
            order[i] = [j for j in range(n_kv) if tile_visible(i, j, r, causal)]
        return order
    seqs = items(schedule, mask, n_q, n_kv)
    G = ring if ring else len(seqs)
    if len(seqs) % G != 0:
        raise ValueError(f"ring {G} does not divide {len(seqs)} items")
    contrib: Dict[int, List[Tuple[int, int, int]]] = {i: [] for i in range(n_q)}
    for it, seq in enumerate(seqs):
        for step, (i, j) in enumerate(seq):
            contrib[i].append((it // G, step, j))
    for i, lst in contrib.items():
        keys = [(k, s) for k, s, _ in lst]
        assert len(set(keys)) == len(keys), f"two contributions to dQ tile {i} at one step of one round"
        order[i] = [j for _, _, j in sorted(lst)]
    return order


def rank_table(schedule: str, mask: str, n_q: int, n_kv: int, ring: int = 0) -> Dict[Tile, int]:
    """(i, j) -> position of KV tile j in dQ tile i's accumulation order."""
    out: Dict[Tile, int] = {}
    for i, js in accumulation_order(schedule, mask, n_q, n_kv, ring).items():
        for pos, j in enumerate(js):
            out[(i, j)] = pos
    return out
