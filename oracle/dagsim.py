"""DAG model of the deterministic attention backward and an exact critical-path simulator.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Model (DASH, zskr.cn explainer section 2.2; gist.science summary section 2.1):
the backward is a directed acyclic graph whose nodes are compute (C) and
reduce (R) stages and whose edges are zero-weight dependencies or positive
weights carrying computation time; the goal is the shortest critical path.
Here every node is an *event* (a stage starting or ending), every edge carries
a weight, and the depth of an event is the longest path reaching it, i.e. its
earliest time. For one tile (i, j):

    Cs --c--> Ce --0--> Rs --r--> Re

The reduce of (i, j) may start only after the reduce of dQ tile i's previous
contributor has ended (edge Re(prev) --0--> Rs), and an SM runs one tile at a
time (edge Re(previous tile on that SM) --0--> Cs): a reduce that waits holds
its SM, because the KV tile's work stays contiguous on one SM.

Closed forms the pages give for m heads on n SMs with n tiles per side
(c = compute cost of a tile, r = reduce cost):
    serial ascending, causal   m*n*(c+r) + (n-1)*r
    descending Q, causal       ~ m*(n+1)*(c+r)/2 + (n-1)*r
    shift, full                m*n*(c+r)
    symmetric shift, causal    m*(n+1)*(c+r)/2
(zskr.cn sections 3.1, 3.2, 3.3). The tests check the simulator against them.

Placement readings (the pages leave them open):
* serial ascending and descending Q dispatch items in (head, KV tile) order to
  the SM that becomes free first, ties to the lower SM id: the descending order
  is said to free resources for the following heads sooner (zskr.cn 3.1).
* shift puts KV tile j of every head on SM j; heads follow each other.
* symmetric shift puts the n/2 pair items of two heads side by side on n SMs.
"""
from collections import defaultdict, deque
from fractions import Fraction
from typing import Dict, Hashable, List, Optional, Tuple

from . import schedules as S


class EventDAG:
    """Edge-weighted DAG over hashable event ids; depth = longest path from any source."""

    def __init__(self):
        self.succ: Dict[Hashable, List[Tuple[Hashable, object]]] = defaultdict(list)
        self.pred: Dict[Hashable, List[Tuple[Hashable, object]]] = defaultdict(list)
        self.nodes: Dict[Hashable, None] = {}

    def add_node(self, v):
        self.nodes.setdefault(v, None)

    def add_edge(self, u, v, w):
        self.add_node(u)
        self.add_node(v)
        self.succ[u].append((v, w))
        self.pred[v].append((u, w))

    def topo_order(self) -> List[Hashable]:
        indeg = {v: len(self.pred[v]) for v in self.nodes}
        q = deque(v for v in self.nodes if indeg[v] == 0)
        order = []
        while q:
            u = q.popleft()
            order.append(u)
            for v, _ in self.succ[u]:
                indeg[v] -= 1
                if indeg[v] == 0:
                    q.append(v)
        if len(order) != len(self.nodes):
            raise ValueError("graph has a cycle")
        return order

    def depths(self) -> Dict[Hashable, object]:
        d: Dict[Hashable, object] = {}
        for v in self.topo_order():
            best = 0
            for u, w in self.pred[v]:
                if d[u] + w > best:
                    best = d[u] + w
            d[v] = best
        return d

    def reaches(self, a, b) -> bool:
        """True if there is a path a -> ... -> b (a == b counts)."""
        seen = {a}
        stack = [a]
        while stack:
            u = stack.pop()
            if u == b:
                return True
            for v, _ in self.succ[u]:
                if v not in seen:
                    seen.add(v)
                    stack.append(v)
        return False

    def critical_path(self):
        d = self.depths()
        return max(d.values()) if d else 0


def _add_tile(g: EventDAG, h, i, j, c, r):
    cs, ce, rs, re = ("Cs", h, i, j), ("Ce", h, i, j), ("Rs", h, i, j), ("Re", h, i, j)
    g.add_edge(cs, ce, c)
    g.add_edge(ce, rs, 0)
    g.add_edge(rs, re, r)
    return cs, re


def build(schedule: str, mask: str, n: int, m: int, c, r, n_sm: Optional[int] = None):
    """Build the event DAG for m heads, n Q tiles = n KV tiles per head, n_sm SMs (default n).

    Returns (dag, assignment) where assignment maps (head, item index) -> SM.
    """
    n_sm = n if n_sm is None else n_sm
    its = S.items(schedule, mask, n, n)
    order = S.accumulation_order(schedule, mask, n, n) if schedule != "atomic_nondet" else None
    rank = {}
    if order is not None:
        for i, js in order.items():
            for pos, j in enumerate(js):
                rank[(i, j)] = pos
    g = EventDAG()
    assignment: Dict[Tuple[int, int], int] = {}
    last_on_sm: Dict[int, Hashable] = {}

    def chain_item(h, it_idx, sm):
        assignment[(h, it_idx)] = sm
        for (i, j) in its[it_idx]:
            cs, re = _add_tile(g, h, i, j, c, r)
            if sm in last_on_sm:
                g.add_edge(last_on_sm[sm], cs, 0)
            last_on_sm[sm] = re
            if order is not None and rank[(i, j)] > 0:
                jp = order[i][rank[(i, j)] - 1]
                g.add_edge(("Re", h, i, jp), ("Rs", h, i, j), 0)

    if schedule in ("serial_ascending", "descending_q", "atomic_nondet"):
        # Greedy: items in (head, KV tile) order to the earliest-free SM, ties to the
        # lower id. An item's rank predecessors belong to earlier items of its head,
        # so every depth it needs is final when it is placed.
        free_at = {s: 0 for s in range(n_sm)}
        for h in range(m):
            for it_idx in range(len(its)):
                sm = min(range(n_sm), key=lambda s: (free_at[s], s))
                chain_item(h, it_idx, sm)
                free_at[sm] = g.depths()[last_on_sm[sm]]
    elif schedule == "shift":
        assert n_sm == n
        for h in range(m):
            for it_idx in range(len(its)):
                chain_item(h, it_idx, it_idx)
    elif schedule == "symmetric_shift":
        assert n_sm == n and m % 2 == 0 and n % 2 == 0
        half = n // 2
        for h in range(m):
            base = 0 if h % 2 == 0 else half
            for it_idx in range(len(its)):
                chain_item(h, it_idx, base + it_idx)
    else:
        raise ValueError(schedule)
    return g, assignment


def makespan(schedule: str, mask: str, n: int, m: int, c, r, n_sm: Optional[int] = None):
    g, _ = build(schedule, mask, n, m, c, r, n_sm)
    return g.critical_path()


def closed_form(schedule: str, mask: str, n: int, m: int, c, r):
    """The pages' closed forms (zskr.cn sections 3.1-3.3); full-mask serial is derived."""
    c, r = Fraction(c), Fraction(r)
    if schedule == "shift" and mask == "full":
        return m * n * (c + r)
    if schedule == "serial_ascending" and mask == "causal":
        return m * n * (c + r) + (n - 1) * r
    if schedule == "descending_q" and mask == "causal":
        return m * (n + 1) * (c + r) / 2 + (n - 1) * r
    if schedule == "symmetric_shift" and mask == "causal":
        return m * (n + 1) * (c + r) / 2
    if schedule in ("serial_ascending", "descending_q") and mask == "full":
        return m * n * (c + r) + (n - 1) * r
    raise ValueError((schedule, mask))


def timeline(schedule: str, mask: str, n: int, m: int, c, r, n_sm: Optional[int] = None):
    """Per-SM schedule of the model: {sm: [(start, compute_end, reduce_start, end, head, i, j), ...]}
    in start order, from the event depths (earliest times). A gap between
    compute_end and reduce_start is the tile's wait for its turn in the dQ order."""
    g, assignment = build(schedule, mask, n, m, c, r, n_sm)
    d = g.depths()
    its = S.items(schedule, mask, n, n)
    per: Dict[int, list] = defaultdict(list)
    for (h, it_idx), sm in assignment.items():
        for (i, j) in its[it_idx]:
            per[sm].append((d[("Cs", h, i, j)], d[("Ce", h, i, j)], d[("Rs", h, i, j)], d[("Re", h, i, j)], h, i, j))
    for sm in per:
        per[sm].sort()
    return dict(per)


def render(per, unit=1) -> str:
    """Text figure of a timeline: one row per SM, one character per `unit` of
    time; a computing tile shows its Q tile index (base 36), its reduce 'r', a
    wait for the dQ turn '.', an idle SM ' '."""
    end = max(t[3] for tl in per.values() for t in tl)
    width = int(-(-end // unit))
    rows = []
    digits = "0123456789abcdefghijklmnopqrstuvwxyz"
    for sm in sorted(per):
        row = [" "] * width
        for (s, ce, rs, e, h, i, j) in per[sm]:
            for x in range(int(s // unit), int(-(-ce // unit))):
                row[x] = digits[i % 36]
            for x in range(int(ce // unit), int(-(-rs // unit))):
                row[x] = "."
            for x in range(int(rs // unit), int(-(-e // unit))):
                row[x] = "r"
        rows.append(f"SM{sm:<3d}|" + "".join(row) + "|")
    return "\n".join(rows)
