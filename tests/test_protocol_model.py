"""CPU model of the ordered dQ hand-off (tests/protocol_model.cpp): threads
stand in for workgroups, atomics for the flags. The items' walks and ranks come
from the library's host view of the device walk (detattn_schedule_item); the
dispatch follows the kernel (ticket counter, or rings in rounds with snake
order). Every run must end, and every dQ tile must hold the fp32 sum of its
partials in rank order, bit for bit; a withheld signal or a ring without all
its workgroups must end in a reported timeout instead of a hang."""
import os
import subprocess

import numpy as np
import pytest

import deterministic_attention_backward_fa_amd as da

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("protocol") / "protocol_model")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", os.path.join(HERE, "protocol_model.cpp"), "-o", exe],
                   check=True)
    return exe


def partial(h, item, t):
    """The model's partial of (head, item, step), as an exact float32."""
    m = 0xFFFFFFFF
    x = ((h * 0x9E3779B1) ^ ((item + 1) * 0x85EBCA77) ^ ((t + 7) * 0xC2B2AE3D)) & m
    x ^= x >> 15
    x = (x * 0x2C1B3C6D) & m
    x ^= x >> 12
    mant = np.float32(1.0) + np.float32(x & 0x7FFFFF) / np.float32(1 << 23)
    v = np.float32(np.ldexp(mant, int((x >> 23) % 8) - 4))
    return -v if x >> 31 else v


def run_model(exe, sched, causal, n_kv, r, BH, mode, G=0, rings=0, snake=False, threads=1, seed=1, drop=-1,
              timeout_ms=20000):
    n_q = n_kv * r
    ip = da.detattn_schedule_items_per_head(sched, causal, n_q, n_kv)
    walks = [da.detattn_schedule_item(sched, causal, n_q, n_kv, it, ring=G if mode == 1 and sched in (
        "shift", "symmetric_shift") else 0) for it in range(ip)]
    lines = [f"{BH} {ip} {n_q} {mode} {G or 1} {rings or 1} {int(snake)} {threads} {seed} {drop} {timeout_ms}"]
    for wk in walks:
        lines.append(" ".join([str(len(wk))] + [f"{i} {rk}" for i, _, rk in wk]))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    res = out.stdout.split()
    return res[0], res[1:], walks, ip, n_q


def expected_bits(walks, BH, n_q):
    contrib = {}
    for h in range(BH):
        for it, wk in enumerate(walks):
            for t, (i, _, rk) in enumerate(wk):
                contrib.setdefault((h, i), []).append((rk, partial(h, it, t)))
    bits = []
    for h in range(BH):
        for i in range(n_q):
            lst = sorted(contrib[(h, i)])
            assert [rk for rk, _ in lst] == list(range(len(lst)))   # ranks are a bijection onto 0..n-1
            acc = lst[0][1]
            for _, v in lst[1:]:
                acc = np.float32(acc + v)
            bits.append(f"{np.array(acc, dtype=np.float32).view(np.uint32):08x}")
    return bits


CASES = []
for sched, causal in (("serial_ascending", False), ("serial_ascending", True), ("descending_q", False),
                      ("descending_q", True), ("shift", False), ("symmetric_shift", True)):
    for n_kv, r in ((4, 1), (8, 2), (8, 1)):
        items = n_kv // 2 if sched == "symmetric_shift" else n_kv
        if sched in ("serial_ascending", "descending_q"):
            for threads in (1, 3, 8):
                CASES.append((sched, causal, n_kv, r, 0, 0, 0, threads))
        for G in sorted({items, max(1, items // 2), 2 if items % 2 == 0 else 1}):
            rings = 2
            CASES.append((sched, causal, n_kv, r, 1, G, rings, G * rings))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{'c' if c[1] else 'f'}-n{c[2]}r{c[3]}-"
                         + (f"ticket{c[7]}" if c[4] == 0 else f"ring{c[5]}x{c[6]}"))
def test_model_ends_with_rank_order_bits(model, case):
    sched, causal, n_kv, r, mode, G, rings, threads = case
    snake = mode == 1 and causal and sched == "descending_q"   # as the library dispatches it
    BH = 3
    for seed in (1, 2, 3):
        status, bits, walks, ip, n_q = run_model(model, sched, causal, n_kv, r, BH, mode, G, rings, snake, threads,
                                                 seed)
        assert status == "OK", (case, seed)
        assert bits == expected_bits(walks, BH, n_q), (case, seed)


def test_snake_order_keeps_the_bits(model):
    """Which workgroup runs an item never changes the order: plain and snake rings agree."""
    a = run_model(model, "descending_q", True, 8, 2, 3, 1, 2, 2, False, 4, seed=5)
    b = run_model(model, "descending_q", True, 8, 2, 3, 1, 2, 2, True, 4, seed=6)
    assert a[0] == b[0] == "OK" and a[1] == b[1]


@pytest.mark.parametrize("sched,causal,mode", [("serial_ascending", False, 0), ("shift", False, 1),
                                               ("symmetric_shift", True, 1)])
def test_withheld_signal_times_out(model, sched, causal, mode):
    G = 4 if mode == 1 else 0
    status, _, _, _, _ = run_model(model, sched, causal, 8, 1, 2, mode, G, 1, False, 4, seed=9, drop=0,
                                   timeout_ms=300)
    assert status == "TIMEOUT"


def test_ring_without_all_its_workgroups_times_out(model):
    """A ring must be co-resident: with only 2 of its 4 workgroups running, the
    missing slots' partials never arrive and the waits expire."""
    status, _, _, _, _ = run_model(model, "shift", False, 4, 1, 1, 1, 4, 1, False, 2, seed=3, timeout_ms=300)
    assert status == "TIMEOUT"


def test_partials_make_the_order_visible():
    """With these partials a wrong summation order changes the bits of many dQ
    tiles (a float sum in another order may still round alike, so not all), so
    the bitwise check above does test the order."""
    walks = [da.detattn_schedule_item("shift", False, 8, 8, it) for it in range(8)]
    want = expected_bits(walks, 2, 8)
    changed = set()
    for perm in (lambda rk: 7 - rk, lambda rk: (rk + 1) % 8):
        other = expected_bits([[(i, j, perm(rk)) for i, j, rk in wk] for wk in walks], 2, 8)
        diff = {x for x, (a, b) in enumerate(zip(want, other)) if a != b}
        assert len(diff) >= 5
        changed |= diff
    assert len(changed) >= 12


def test_thousand_interleavings(model):
    """1000 seeded interleavings across the dispatch forms, each ending with the
    rank-order bits."""
    configs = [("serial_ascending", True, 4, 2, 0, 0, 0, 3), ("descending_q", True, 4, 2, 1, 2, 2, 4),
               ("shift", False, 4, 1, 1, 2, 2, 4), ("symmetric_shift", True, 4, 2, 1, 1, 2, 2)]
    want = {}
    for seed in range(1000):
        sched, causal, n_kv, r, mode, G, rings, threads = configs[seed % 4]
        snake = mode == 1 and causal and sched == "descending_q"
        status, bits, walks, _, n_q = run_model(model, sched, causal, n_kv, r, 2, mode, G, rings, snake, threads,
                                                seed)
        assert status == "OK", (sched, seed)
        key = seed % 4
        if key not in want:
            want[key] = expected_bits(walks, 2, n_q)
        assert bits == want[key], (sched, seed)
