"""Pins of the oracle's schedule definitions: golden n = 4 tables, exact coverage,
conflict-free steps, and the pages' load-balance claims."""
import json
import os

import pytest

from oracle import schedules as S

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "schedules_n4.json")))


def test_golden_shift_n4():
    g = GOLDEN["shift_full"]
    its = S.items("shift", "full", 4, 4)
    assert [[i for i, _ in it] for it in its] == g["visits_q_tiles_per_kv_tile"]
    assert {str(k): v for k, v in S.accumulation_order("shift", "full", 4, 4).items()} == g["dq_order"]


def test_golden_symmetric_n4():
    g = GOLDEN["symmetric_shift_causal"]
    its = S.items("symmetric_shift", "causal", 4, 4)
    assert [[list(t) for t in it] for it in its] == g["items_tiles_q_kv"]
    assert all(len(it) == g["tiles_per_item"] for it in its)
    assert {str(k): v for k, v in S.accumulation_order("symmetric_shift", "causal", 4, 4).items()} == g["dq_order"]


@pytest.mark.parametrize("name,sched", [("serial_ascending_causal", "serial_ascending"),
                                        ("descending_q_causal", "descending_q")])
def test_golden_serial_and_descending_n4(name, sched):
    g = GOLDEN[name]
    its = S.items(sched, "causal", 4, 4)
    assert [[i for i, _ in it] for it in its] == g["visits_q_tiles_per_kv_tile"]
    assert {str(k): v for k, v in S.accumulation_order(sched, "causal", 4, 4).items()} == g["dq_order"]


CASES = [(n_kv, r) for n_kv in (2, 4, 6, 8, 16) for r in (1, 2, 4)]


@pytest.mark.parametrize("n_kv,r", CASES)
@pytest.mark.parametrize("sched,mask", [("serial_ascending", "full"), ("serial_ascending", "causal"),
                                        ("descending_q", "full"), ("descending_q", "causal"),
                                        ("shift", "full"), ("symmetric_shift", "causal"),
                                        ("atomic_nondet", "full"), ("atomic_nondet", "causal")])
def test_exact_once_coverage(sched, mask, n_kv, r):
    n_q = n_kv * r
    its = S.items(sched, mask, n_q, n_kv)
    seen = [t for it in its for t in it]
    want = [(i, j) for i in range(n_q) for j in range(n_kv) if S.tile_visible(i, j, r, mask == "causal")]
    assert sorted(seen) == sorted(want) and len(seen) == len(set(seen))


@pytest.mark.parametrize("n_kv,r", CASES)
def test_shift_and_symmetric_are_conflict_free(n_kv, r):
    # At every lock-step the items touch pairwise distinct dQ tiles, so no item ever
    # has to wait for a concurrent one (zskr.cn 3.2 'conflict-free reduction').
    n_q = n_kv * r
    for sched, mask in (("shift", "full"), ("symmetric_shift", "causal")):
        its = S.items(sched, mask, n_q, n_kv)
        L = len(its[0])
        assert all(len(it) == L for it in its), "unequal item lengths break the lock step"
        for t in range(L):
            rows = [it[t][0] for it in its]
            assert len(set(rows)) == len(rows), (sched, t, rows)


@pytest.mark.parametrize("n_kv,r", CASES)
def test_symmetric_items_are_balanced(n_kv, r):
    # Folding the triangle into a rectangle: every pair holds n_q + r tiles (r = 1: N + 1).
    n_q = n_kv * r
    its = S.items("symmetric_shift", "causal", n_q, n_kv)
    assert all(len(it) == n_q + r for it in its)
    for p, it in enumerate(its):
        assert {j for _, j in it} == {p, n_kv - 1 - p}


def test_descending_keeps_the_ascending_dq_order():
    for mask in ("full", "causal"):
        assert S.accumulation_order("descending_q", mask, 8, 4) == S.accumulation_order("serial_ascending", mask, 8, 4)


def test_invalid_pairs():
    assert not S.valid("shift", "causal", 8, 8)
    assert not S.valid("symmetric_shift", "full", 8, 8)
    assert not S.valid("symmetric_shift", "causal", 5, 5)
    with pytest.raises(ValueError):
        S.items("shift", "causal", 4, 4)


def test_golden_rings_n4():
    g = GOLDEN["rings"]
    got = S.accumulation_order("shift", "full", 4, 4, ring=2)
    assert {str(k): v for k, v in got.items()} == g["shift_full_G2"]["dq_order"]
    got = S.accumulation_order("symmetric_shift", "causal", 4, 4, ring=1)
    assert {str(k): v for k, v in got.items()} == g["symmetric_shift_causal_G1"]["dq_order"]


@pytest.mark.parametrize("n_kv,r", [(4, 1), (8, 2), (16, 1), (16, 2)])
def test_ring_orders_reduce_to_plain_cases(n_kv, r):
    """One item per round orders every dQ tile by item index (inside a
    symmetric pair: its left column, then its right one); a ring as large as
    the item count is the pages' single round."""
    n_q = n_kv * r
    shift1 = S.accumulation_order("shift", "full", n_q, n_kv, ring=1)
    assert all(js == list(range(n_kv)) for js in shift1.values())
    assert S.accumulation_order("shift", "full", n_q, n_kv, ring=n_kv) == S.accumulation_order(
        "shift", "full", n_q, n_kv)
    sym1 = S.accumulation_order("symmetric_shift", "causal", n_q, n_kv, ring=1)
    for i, js in sym1.items():
        want = []
        for p in range(n_kv // 2):
            want += [j for j in (p, n_kv - 1 - p) if S.tile_visible(i, j, r, True)]
        assert js == want
    P = n_kv // 2
    assert S.accumulation_order("symmetric_shift", "causal", n_q, n_kv, ring=P) == S.accumulation_order(
        "symmetric_shift", "causal", n_q, n_kv)


@pytest.mark.parametrize("n_kv,r", [(8, 1), (16, 2), (32, 1)])
def test_ring_orders_cover_each_contribution_once(n_kv, r):
    n_q = n_kv * r
    for sched, mask, ip in (("shift", "full", n_kv), ("symmetric_shift", "causal", n_kv // 2)):
        for G in [g for g in range(1, ip + 1) if ip % g == 0]:
            order = S.accumulation_order(sched, mask, n_q, n_kv, ring=G)
            for i, js in order.items():
                assert sorted(js) == [j for j in range(n_kv) if S.tile_visible(i, j, r, mask == "causal")]
    with pytest.raises(ValueError):
        S.accumulation_order("shift", "full", 12, 12, ring=5)


@pytest.mark.parametrize("bq,r", [(1, 1), (2, 1), (2, 2), (3, 2), (2, 4)])
def test_tile_visibility_from_the_elementwise_causal_mask(bq, r):
    """A tile pair is visible iff some key position in the KV tile is at or
    before some query position in the Q tile (the causal mask of R3, one
    sequence for queries and keys), counted element by element."""
    bkv = bq * r
    for n_kv in range(1, 6):
        n_q = n_kv * r
        for i in range(n_q):
            for j in range(n_kv):
                brute = any(kv <= q for q in range(i * bq, (i + 1) * bq) for kv in range(j * bkv, (j + 1) * bkv))
                assert S.tile_visible(i, j, r, True) == brute, (bq, r, i, j)
                assert S.tile_visible(i, j, r, False)


@pytest.mark.parametrize("n_kv,r", [(4, 1), (8, 2), (6, 2), (4, 4)])
def test_shift_items_start_at_their_own_index(n_kv, r):
    """Each KV tile's workgroup starts at its own index and wraps around
    (zskr.cn explainer section 3.2, read as R6 for any r): item j's first Q tile
    is j, and the items of one step cover n_kv consecutive Q tiles (cyclically)."""
    n_q = n_kv * r
    its = S.items("shift", "full", n_q, n_kv)
    for j, seq in enumerate(its):
        assert seq[0] == (j, j)
        assert [i for i, _ in seq] == [(j + t) % n_q for t in range(n_q)]
    for t in range(n_q):
        assert sorted((seq[t][0] - t) % n_q for seq in its) == list(range(n_kv))


@pytest.mark.parametrize("n_kv,r", [(4, 1), (8, 2), (6, 2)])
def test_symmetric_phase1_starts_at_the_items_own_index(n_kv, r):
    """Symmetric shift's phase 1 shifts item p over the dense rectangle (Q tiles
    n_q/2.., KV tile p) starting at the rectangle's Q tile p (R7): its first
    n_q/2 tiles are n_q/2 + (p + t) mod n_q/2."""
    n_q = n_kv * r
    half = n_q // 2
    for p, seq in enumerate(S.items("symmetric_shift", "causal", n_q, n_kv)):
        assert seq[:half] == [(half + (p + t) % half, p) for t in range(half)]


@pytest.mark.parametrize("n_kv,r", [(4, 1), (8, 2), (6, 2), (16, 2)])
def test_symmetric_rows_above_the_rectangle_go_by_residue_class(n_kv, r):
    """Phase 2 of item p takes column p's rows above the rectangle, p*r ..
    n_q/2 - 1, upward one residue class mod r after another (R7), then column
    n_kv-1-p's rows downward the same way. Every dQ tile then receives its
    partials in the same order as if the rows were taken plainly upward and
    downward, so the reading changes the visits inside an item, not a dQ tile's
    accumulation order."""
    n_q = n_kv * r
    half = n_q // 2
    its = S.items("symmetric_shift", "causal", n_q, n_kv)
    plain = []
    for p, seq in enumerate(its):
        top = seq[half:half + half - p * r]
        assert top == [(i, p) for k in range(r) for i in range(p * r + k, half, r)]
        rest = seq[half + len(top):]
        c = n_kv - 1 - p
        assert rest == [(i, c) for k in range(r) for i in range(n_q - r + k, c * r - 1, -r)]
        plain.append(seq[:half] + [(i, p) for i in range(p * r, half)] +
                     [(i, c) for i in range(n_q - 1, c * r - 1, -1)])

    def order(items):
        got = {}
        for t in range(max(len(x) for x in items)):
            for x in items:
                if t < len(x):
                    got.setdefault(x[t][0], []).append(x[t][1])
        return got

    assert order(its) == order(plain)
    assert order(its) == S.accumulation_order("symmetric_shift", "causal", n_q, n_kv)
