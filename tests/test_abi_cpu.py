"""Host-side checks of libdetattn that need no GPU.

Every call here returns before anything is enqueued (argument, support and
workspace errors, planning with an explicit grid, the schedule view), so the
file is safe on a machine with or without a GPU; no test passes a fake
pointer to a call that could launch.
"""
import ctypes
import os
import re

import pytest

import deterministic_attention_backward_fa_amd as da
from oracle import schedules as OS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "detattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    names = declared_functions()
    assert "attn_bwd_deterministic" in names and "detattn_fwd" in names and len(names) >= 9
    L = ctypes.CDLL(da.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/detattn.h but not exported"


def test_status_strings():
    for code in range(8):
        assert da.status_string(code) and da.status_string(code) != "unknown status"
    assert da.status_string(99) == "unknown status"


def test_workspace_bytes():
    B, H, S, D = 1, 32, 8192, 128
    n = da.detattn_bwd_workspace_bytes(B, H, S, D)
    # fp32 dQ accumulator + fp32 D + one 128-byte flag line per 64-row Q tile + header, 256-byte aligned
    assert n >= 4 * B * H * S * D + 4 * B * H * S + 128 * B * H * (S // 64) + 256
    assert n % 256 == 0
    assert da.detattn_bwd_workspace_bytes(1, 1, 64, -1) == 0


def _bwd_status(shape, mask=0, sched=0, ptr=0x10000, ws=0x20000, ws_bytes=1 << 40, opts=None):
    L = da.lib()
    p = ctypes.c_void_p(ptr)
    args = [p] * 9 + [ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), da.Shape(*shape), mask, sched]
    if opts is None:
        return L.attn_bwd_deterministic(*args, None)
    return L.attn_bwd_deterministic_ex(*args, ctypes.byref(opts), None)


def test_argument_errors_return_before_launch():
    # null pointers
    assert _bwd_status((1, 1, 128, 64, 0.125), ptr=0) == 1
    # misaligned pointer
    assert _bwd_status((1, 1, 128, 64, 0.125), ptr=0x10008) == 1
    # bad enums
    assert _bwd_status((1, 1, 128, 64, 0.125), mask=7) == 1
    assert _bwd_status((1, 1, 128, 64, 0.125), sched=9) == 1
    # negative size
    assert _bwd_status((1, -1, 128, 64, 0.125)) == 1
    # empty problems are a valid no-op
    assert _bwd_status((0, 4, 128, 64, 0.125)) == 0
    assert _bwd_status((2, 4, 0, 64, 0.125)) == 0


def test_unsupported_configurations():
    # head dimension not built
    assert _bwd_status((1, 1, 128, 96, 0.1)) == 2
    # S not a multiple of the tile
    assert _bwd_status((1, 1, 100, 64, 0.125), opts=da._options(grid=8)) == 2
    # shift is defined for full masks only, symmetric shift for causal masks only
    assert _bwd_status((1, 1, 256, 64, 0.125), mask=1, sched=2, opts=da._options(grid=8)) == 2
    assert _bwd_status((1, 1, 256, 64, 0.125), mask=0, sched=3, opts=da._options(grid=8)) == 2
    # symmetric shift needs an even number of KV tiles (3 tiles of 64 rows)
    assert _bwd_status((1, 1, 192, 64, 0.125), mask=1, sched=3, opts=da._options(grid=8, block_q=64,
                                                                                     block_kv=64)) == 2
    # a tile pair that is not built
    assert _bwd_status((1, 1, 256, 128, 0.1), opts=da._options(grid=8, block_q=128, block_kv=128)) == 2
    # a ring larger than the grid cannot be co-resident
    assert _bwd_status((1, 1, 1024, 64, 0.125), sched=2, opts=da._options(grid=8, block_q=64, block_kv=64)) == 2


def test_workspace_errors():
    o = da._options(grid=8)
    assert _bwd_status((1, 1, 128, 64, 0.125), ws=0, opts=o) == 3
    assert _bwd_status((1, 1, 128, 64, 0.125), ws=0x20010, opts=o) == 3  # not 256-byte aligned
    need = da.detattn_bwd_workspace_bytes(1, 1, 128, 64)
    assert _bwd_status((1, 1, 128, 64, 0.125), ws_bytes=need - 1, opts=o) == 3


def test_fwd_argument_errors():
    L = da.lib()
    p = ctypes.c_void_p(0x10000)
    assert L.detattn_fwd(p, p, p, p, ctypes.c_void_p(0), da.Shape(1, 1, 128, 64, 0.1), 0, None) == 1
    assert L.detattn_fwd(p, p, p, p, p, da.Shape(1, 1, 128, 80, 0.1), 0, None) == 2
    assert L.detattn_fwd(p, p, p, p, p, da.Shape(1, 1, 96, 64, 0.1), 0, None) == 2
    assert L.detattn_fwd(p, p, p, p, p, da.Shape(1, 1, 128, 64, 0.1), 5, None) == 1
    assert L.detattn_fwd(p, p, p, p, p, da.Shape(0, 1, 128, 64, 0.1), 0, None) == 0


@pytest.mark.parametrize("cfg", [
    # (B, H, S, D, causal, schedule, expected block_q, block_kv)
    (1, 2, 256, 64, False, "shift", 64, 64),
    (4, 16, 2048, 64, True, "symmetric_shift", 128, 128),
    (2, 32, 4096, 128, False, "shift", 64, 128),
    (1, 32, 8192, 128, True, "symmetric_shift", 64, 128),
    (1, 16, 16384, 128, False, "shift", 64, 128),           # 128-row KV tiles at 16k too (measured faster)
    (1, 16, 16384, 128, True, "symmetric_shift", 64, 128),
])
def test_default_tiles_and_rings(cfg):
    B, H, S, D, causal, sched, bq, bkv = cfg
    p = da.detattn_bwd_plan(B, H, S, D, causal, sched, grid=256)
    assert (p["block_q"], p["block_kv"]) == (bq, bkv)
    n_kv = S // bkv
    items = n_kv if sched == "shift" else n_kv // 2
    ring = min(items, 32)  # one XCD's workgroups; larger heads take their items in rounds
    assert p["ring"] == ring and p["cooperative"] == 0  # plain launch unless asked
    assert p["grid"] == p["rings"] * ring <= 256
    assert p["rings"] >= 1
    c = da.detattn_bwd_plan(B, H, S, D, causal, sched, grid=256, cooperative_launch=True)
    assert c["cooperative"] == 1 and {k: c[k] for k in c if k != "cooperative"} == \
        {k: p[k] for k in p if k != "cooperative"}


def test_ticket_plan_caps_grid_at_items():
    p = da.detattn_bwd_plan(1, 2, 256, 64, False, "serial_ascending", grid=256, dispatch="ticket")
    assert p["items"] == 2 * 4 and p["grid"] == 8 and p["ring"] == 0 and p["cooperative"] == 0
    p = da.detattn_bwd_plan(1, 2, 256, 64, False, "atomic_nondet", grid=256, dispatch="ticket")
    assert p["grid"] == 8 and p["ring"] == 0 and p["cooperative"] == 0 and p["dq_mode"] == 0


@pytest.mark.parametrize("sched", ["serial_ascending", "descending_q", "atomic_nondet"])
def test_serial_descending_atomic_rings(sched):
    """Serial and descending run on rings of one XCD where one fits (their
    ordered adds stay in that XCD's L2), else on the ticket counter; the
    atomic reference takes rings (adds in one XCD's L2) only when asked."""
    ask = {"dispatch": "ring"} if sched == "atomic_nondet" else {}
    p = da.detattn_bwd_plan(1, 32, 8192, 128, True, sched, grid=256, **ask)
    assert (p["ring"], p["rings"], p["cooperative"], p["dq_mode"]) == (32, 8, 0, da.DQ_MODES["xcd_local"])
    if sched == "atomic_nondet":
        p = da.detattn_bwd_plan(1, 32, 8192, 128, True, sched, grid=256)
        assert (p["ring"], p["cooperative"], p["dq_mode"]) == (0, 0, 0)
    p = da.detattn_bwd_plan(1, 32, 8192, 128, True, sched, grid=100)       # no XCD placement: ticket
    device_mode = 0 if sched == "atomic_nondet" else da.DQ_MODES["atomic"]
    assert (p["ring"], p["cooperative"], p["dq_mode"]) == (0, 0, device_mode)
    p = da.detattn_bwd_plan(1, 32, 8192, 128, True, sched, grid=256, dispatch="ticket", cooperative_launch=True)
    assert (p["ring"], p["cooperative"]) == (0, 0)  # a ticket is only taken by a running workgroup
    p = da.detattn_bwd_plan(1, 32, 8192, 128, True, sched, grid=256, dispatch="ring", ring_size=16)
    assert (p["ring"], p["rings"], p["cooperative"]) == (16, 16, 0)


CASES = [(n_kv, r) for n_kv in (1, 2, 4, 6, 8, 16, 32) for r in (1, 2)]


@pytest.mark.parametrize("n_kv,r", CASES)
@pytest.mark.parametrize("sched,mask", [("serial_ascending", "full"), ("serial_ascending", "causal"),
                                        ("descending_q", "full"), ("descending_q", "causal"),
                                        ("shift", "full"), ("symmetric_shift", "causal"),
                                        ("atomic_nondet", "full"), ("atomic_nondet", "causal")])
def test_library_schedule_matches_oracle(sched, mask, n_kv, r):
    """The library's closed-form visit orders and ranks equal the oracle's
    definitions (built by sorting contributions by step)."""
    n_q = n_kv * r
    causal = mask == "causal"
    if not OS.valid(sched, mask, n_q, n_kv):
        assert da.detattn_schedule_items_per_head(sched, causal, n_q, n_kv) == -1
        return
    want_items = OS.items(sched, mask, n_q, n_kv)
    assert da.detattn_schedule_items_per_head(sched, causal, n_q, n_kv) == len(want_items)
    ranks = OS.rank_table(sched, mask, n_q, n_kv) if sched != "atomic_nondet" else None
    for it, want in enumerate(want_items):
        got = da.detattn_schedule_item(sched, causal, n_q, n_kv, it)
        assert [(a, b) for a, b, _ in got] == want
        if ranks is not None:
            assert [c for _, _, c in got] == [ranks[t] for t in want]


RING_CASES = [(n_kv, r) for n_kv in (4, 6, 8, 12, 16, 64, 128) for r in (1, 2)]


@pytest.mark.parametrize("n_kv,r", RING_CASES)
@pytest.mark.parametrize("sched,mask", [("shift", "full"), ("symmetric_shift", "causal")])
def test_library_ring_ranks_match_oracle(sched, mask, n_kv, r):
    """With a ring of G workgroups the library's ranks (the incremental walk the
    kernel takes, checked in the library against its counting closed form)
    equal the oracle's round-major order, for every divisor G of the items."""
    n_q = n_kv * r
    causal = mask == "causal"
    ip = da.detattn_schedule_items_per_head(sched, causal, n_q, n_kv)
    want_items = OS.items(sched, mask, n_q, n_kv)
    rings = [g for g in range(1, ip + 1) if ip % g == 0]
    if n_kv >= 64:
        rings = [g for g in rings if g in (1, 2, 8, 32, ip)]
    for G in rings:
        ranks = OS.rank_table(sched, mask, n_q, n_kv, ring=G)
        for it, want in enumerate(want_items):
            got = da.detattn_schedule_item(sched, causal, n_q, n_kv, it, ring=G)
            assert [(a, b) for a, b, _ in got] == want
            assert [c for _, _, c in got] == [ranks[t] for t in want], (G, it)
    bad = [g for g in range(2, ip) if ip % g != 0]
    for G in bad[:2]:
        with pytest.raises(da.DetAttnError):
            da.detattn_schedule_item(sched, causal, n_q, n_kv, 0, ring=G)


def test_ring_option_in_plan():
    """Default rings at these shapes: a head's items if they fit one XCD (32
    workgroups), else 32 (items in rounds); an explicit ring_size must divide
    the items."""
    kv64 = dict(block_q=64, block_kv=64)
    p = da.detattn_bwd_plan(1, 16, 16384, 128, True, "symmetric_shift", grid=256, **kv64)
    assert (p["n_kv"], p["ring"], p["rings"], p["grid"]) == (256, 32, 8, 256)
    p = da.detattn_bwd_plan(1, 16, 16384, 128, False, "shift", grid=256, **kv64)
    assert (p["ring"], p["rings"], p["dq_mode"]) == (32, 8, da.DQ_MODES["xcd_local"])
    p = da.detattn_bwd_plan(1, 16, 16384, 128, True, "symmetric_shift", grid=256)
    assert (p["n_kv"], p["ring"], p["rings"]) == (128, 32, 8)
    p = da.detattn_bwd_plan(1, 32, 8192, 128, True, "symmetric_shift", grid=256)
    assert (p["ring"], p["rings"]) == (32, 8)
    p = da.detattn_bwd_plan(1, 16, 16384, 128, False, "shift", grid=256, ring_size=256, **kv64)
    assert (p["ring"], p["rings"], p["dq_mode"]) == (256, 1, da.DQ_MODES["atomic"])
    with pytest.raises(da.DetAttnError):
        da.detattn_bwd_plan(1, 16, 16384, 128, False, "shift", grid=256, ring_size=48, **kv64)


@pytest.mark.parametrize("H,S,D,causal,grid,want", [
    (2, 4096, 128, False, 256, "shift"), (2, 8192, 128, True, 256, "symmetric_shift"),
    (2, 16384, 128, True, 256, "descending_q"),
    (2, 4096, 128, True, 256, "symmetric_shift"), (2, 8192, 64, True, 256, "symmetric_shift"),
    (2, 2048, 64, True, 256, "symmetric_shift"), (16, 16384, 128, False, 256, "shift"),
    (2, 4096, 128, False, 100, "shift"),
    (2, 384, 128, True, 256, "descending_q"),                        # 3 KV tiles: no symmetric pairing
    (2, 192, 128, True, 256, "descending_q"),                        # 64-row KV tiles (S % 128 != 0), 3 of them
    (2, 16384, 128, False, 256, "shift"),
])
def test_auto_schedule_resolves_from_the_shape(H, S, D, causal, grid, want):
    p = da.detattn_bwd_plan(1, H, S, D, causal, "auto", grid=grid)
    assert da.SCHEDULE_NAMES[p["schedule"]] == want
    q = da.detattn_bwd_plan(1, H, S, D, causal, want, grid=grid)
    assert p == q


@pytest.mark.parametrize("H,n_kv", [(16, 37), (32, 37), (16, 40), (32, 40), (1, 64), (3, 37)])
@pytest.mark.parametrize("sched,causal", [("serial_ascending", False), ("descending_q", False), ("shift", False),
                                          ("serial_ascending", True), ("descending_q", True),
                                          ("symmetric_shift", True), ("auto", False), ("auto", True)])
def test_plans_keep_the_chip_busy_at_any_length(H, n_kv, sched, causal):
    """Sequence lengths whose tile counts are not powers of two (a prime count
    of 128-row KV tiles, say): whatever the divisors of the item count, the
    default plan's makespan in item times (a ring's heads one after the other,
    items / G rounds each; twice as long per item on a ring spanning XCDs, 1.8x
    on the ticket counter, the measured costs of device-scope dQ adds) stays
    within 2.5x the ideal of all items spread over 256 workgroups (ring sizes
    must divide the item count: a prime count of 37 items per head leaves one
    ring of 37 workgroups spanning XCDs, six at a time)."""
    S = n_kv * 128
    if sched == "symmetric_shift" and n_kv % 2:
        with pytest.raises(da.DetAttnError):
            da.detattn_bwd_plan(1, H, S, 128, causal, sched, grid=256)
        return
    p = da.detattn_bwd_plan(1, H, S, 128, causal, sched, grid=256)
    items_per_head = p["items"] // H
    ideal = -(-p["items"] // 256)
    if p["ring"]:
        rounds = -(-H // min(p["rings"], H)) * (items_per_head // p["ring"])
        cost = rounds * (1.0 if p["dq_mode"] == da.DQ_MODES["xcd_local"] else 2.0)
    else:
        cost = -(-p["items"] // p["grid"]) * 1.8
    assert cost <= 2.5 * ideal, p


def test_default_ring_depends_on_the_shape_only():
    """The shift schedules' default ring size sets the dQ order, so it must not
    follow the grid: the same G with any grid."""
    for causal, sched in ((False, "shift"), (True, "symmetric_shift")):
        for H, S in ((16, 4736 * 2), (32, 5120), (1, 16384), (32, 8192)):
            rings = {da.detattn_bwd_plan(1, H, S, 128, causal, sched, grid=g)["ring"] for g in (256, 248, 512)}
            assert len(rings) == 1, (sched, H, S, rings)


def test_shape_bounds_for_32_bit_offsets():
    """One head's fp32 dQ accumulator (S*D*4 bytes) must stay below 2^31."""
    assert _bwd_status((1, 1, (1 << 22), 128, 0.1), opts=da._options(grid=8)) == 1   # S*D*4 = 2^31
    assert _bwd_status((1, 1, (1 << 22) - 64, 128, 0.1), opts=da._options(grid=8)) != 1
    assert da.detattn_bwd_workspace_bytes(1, 1, 1 << 22, 128) == 0


def test_noalloc_entry_refuses_before_any_hip_call():
    """attn_bwd_deterministic_noalloc checks the shape against its fixed scratch
    first: too large a shape is DETATTN_ERR_SCRATCH_LIMIT, an invalid one
    INVALID_ARG, with no device in reach; the no-alloc status needs a device
    that has run the entry point."""
    L = da.lib()
    p = ctypes.c_void_p(0x10000)
    assert L.attn_bwd_deterministic_noalloc(p, p, p, p, p, p, p, p, p, da.Shape(1, 64, 8192, 128, 0.088), 1, 3,
                                            None) == 7
    assert L.attn_bwd_deterministic_noalloc(p, p, p, p, p, p, p, p, p, da.Shape(1, -1, 8192, 128, 0.088), 1, 3,
                                            None) == 1
    # the largest workload shapes here fit: B*H*S*D = 2^25
    assert da.detattn_bwd_workspace_bytes(1, 32, 8192, 128) <= da.NOALLOC_SCRATCH_BYTES
    assert da.detattn_bwd_workspace_bytes(4, 16, 8192, 64) <= da.NOALLOC_SCRATCH_BYTES


def test_resident_pair_option():
    """pair_columns selects the resident-pair form of symmetric shift, built at
    D = 64 with 64 x 64 tiles; other schedules, tiles or head dimensions are
    UNSUPPORTED."""
    kv64 = dict(block_q=64, block_kv=64, grid=256)
    p = da.detattn_bwd_plan(1, 2, 1024, 64, True, "symmetric_shift", pair_columns=True, **kv64)
    assert p["pair_columns"] == 1 and p["schedule"] == da.SCHEDULES["symmetric_shift"]
    assert da.detattn_bwd_plan(1, 2, 1024, 64, True, "symmetric_shift", **kv64)["pair_columns"] == 0
    for args, kw in [((1, 2, 1024, 64, True, "descending_q"), kv64),
                     ((1, 2, 1024, 64, True, "symmetric_shift"), dict(grid=256)),     # 128 x 128 tiles
                     ((1, 2, 1024, 128, True, "symmetric_shift"), kv64)]:            # D = 128: does not fit
        with pytest.raises(da.DetAttnError):
            da.detattn_bwd_plan(*args, pair_columns=True, **kw)
