"""Pins of the DAG simulator: the pages' closed forms and Lemma 1."""
import random
from fractions import Fraction

import pytest

from oracle import dagsim as G

CASES = [(4, 2, 3, 1), (4, 4, 3, 2), (8, 6, 5, 2), (8, 4, 2, 2), (16, 4, 7, 3), (6, 4, 5, 1), (4, 2, 1, 1)]


@pytest.mark.parametrize("n,m,c,r", CASES)
@pytest.mark.parametrize("sched,mask", [("shift", "full"), ("serial_ascending", "causal"),
                                        ("descending_q", "causal"), ("symmetric_shift", "causal"),
                                        ("serial_ascending", "full"), ("descending_q", "full")])
def test_closed_forms(sched, mask, n, m, c, r):
    # zskr.cn explainer 3.1 (T_causal, T_reversed), 3.2 (T_full_opt), 3.3 (T_causal_opt).
    # The full-mask serial form is derived in the same model.
    assert G.makespan(sched, mask, n, m, c, r) == G.closed_form(sched, mask, n, m, c, r)


def test_fractional_costs():
    c, r = Fraction(7, 3), Fraction(1, 2)
    assert G.makespan("shift", "full", 6, 2, c, r) == G.closed_form("shift", "full", 6, 2, c, r)
    assert G.makespan("symmetric_shift", "causal", 6, 2, c, r) == G.closed_form("symmetric_shift", "causal", 6, 2, c, r)


def test_descending_beats_serial_and_symmetric_is_optimal():
    # The orderings the pages claim for causal masks (zskr.cn 3.1 and 3.3).
    for n, m, c, r in CASES:
        ser = G.makespan("serial_ascending", "causal", n, m, c, r)
        desc = G.makespan("descending_q", "causal", n, m, c, r)
        sym = G.makespan("symmetric_shift", "causal", n, m, c, r)
        assert sym <= desc <= ser
        # symmetric shift leaves no idle time: total work / n SMs
        total = m * n * (n + 1) // 2 * (c + r)
        assert sym * n == total


def test_shift_has_no_bubbles():
    for n, m, c, r in CASES:
        assert G.makespan("shift", "full", n, m, c, r) * n == m * n * n * (c + r)


def _random_dag(rng, nn, p):
    g = G.EventDAG()
    for v in range(nn):
        g.add_node(v)
    for u in range(nn):
        for v in range(u + 1, nn):
            if rng.random() < p:
                g.add_edge(u, v, rng.choice([0, 0, 1, 2, 3, 5]))
    return g


def test_lemma1_zero_weight_edge():
    # gist.science summary 2.2B: adding a zero-weight edge u -> v keeps the DAG's
    # depths iff depth(u) <= depth(v). Checked on every admissible pair of many
    # random DAGs, in both directions of the equivalence.
    rng = random.Random(1234)
    checked = {True: 0, False: 0}
    for trial in range(60):
        g = _random_dag(rng, rng.randint(4, 9), 0.35)
        base = g.depths()
        for u in list(g.nodes):
            for v in list(g.nodes):
                if u == v or g.reaches(v, u):
                    continue  # the edge would close a cycle
                h = G.EventDAG()
                for a in g.nodes:
                    h.add_node(a)
                for a in g.nodes:
                    for b, w in g.succ[a]:
                        h.add_edge(a, b, w)
                h.add_edge(u, v, 0)
                unchanged = h.depths() == base
                assert unchanged == (base[u] <= base[v])
                checked[unchanged] += 1
    assert checked[True] > 100 and checked[False] > 100


def test_four_sm_timelines_reconstruct_the_shift_figures():
    """The pages illustrate the shift schedule on 4 SMs with a figure that the
    text lost (zskr.cn explainer 3.2; the symmetric form, 3.3). The model's
    timelines at n = 4, m = 2, c = 3, r = 1: under shift SM j computes Q tiles
    j, j+1, ... (mod 4) of its KV tile, head after head, with no wait; under
    symmetric shift two heads run side by side, each SM holding one pair item of
    n + 1 = 5 tiles back to back (the derived fold: pair p = KV tiles p, 3 - p)."""
    c, r = 3, 1
    per = G.timeline("shift", "full", 4, 2, c, r)
    assert sorted(per) == [0, 1, 2, 3]
    for sm, tl in per.items():
        assert [(h, i, j) for (_, _, _, _, h, i, j) in tl] == [(h, (sm + t) % 4, sm) for h in range(2) for t in range(4)]
        for k, (s, ce, rs, e, *_rest) in enumerate(tl):
            assert (s, ce, rs, e) == (k * (c + r), k * (c + r) + c, k * (c + r) + c, (k + 1) * (c + r))
    fig = G.render(per)
    assert fig.splitlines()[1] == "SM1  |111r222r333r000r111r222r333r000r|"
    per = G.timeline("symmetric_shift", "causal", 4, 2, c, r)
    golden = {0: [(2, 0), (3, 0), (0, 0), (1, 0), (3, 3)], 1: [(3, 1), (2, 1), (1, 1), (3, 2), (2, 2)]}
    for sm, tl in per.items():
        assert [(i, j) for (*_x, h, i, j) in tl] == golden[sm % 2]
        assert all(h == sm // 2 for (*_x, h, i, j) in tl)
        assert [t[0] for t in tl] == [k * (c + r) for k in range(5)]   # no waits, no idle time
