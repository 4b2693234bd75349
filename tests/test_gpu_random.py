"""Randomised GPU parity: seeded random small shapes, schedules and plan options
(tiles, ring sizes, dispatch, dQ mode, grid) against the fp64 oracle, with the
device status checked after every call and a repeat checked bit for bit."""
import math
import random

import pytest

import deterministic_attention_backward_fa_amd as da
from oracle import ref as oref

from gpu_util import TOL, inputs, rel_err, same_bits, say

pytestmark = pytest.mark.gpu

TILES = {64: [(128, 128), (64, 128), (64, 64)], 128: [(64, 128), (64, 64)]}


def draw(rng):
    D = rng.choice([64, 128])
    bq, bkv = rng.choice(TILES[D])
    S = 128 * rng.choice([1, 2, 3, 4, 6, 8])   # the forward that makes O and LSE takes S % 128 == 0
    causal = rng.random() < 0.5
    sched = rng.choice(["serial_ascending", "descending_q", "atomic_nondet", "auto",
                        "symmetric_shift" if causal else "shift"])
    n_kv = S // bkv
    if sched == "symmetric_shift" and n_kv % 2:
        sched = "descending_q"
    opts = {"block_q": bq, "block_kv": bkv}
    items = n_kv // 2 if sched == "symmetric_shift" else n_kv
    if sched in ("shift", "symmetric_shift") or (sched in ("serial_ascending", "descending_q")
                                                  and rng.random() < 0.5):
        opts["ring_size"] = rng.choice([g for g in range(1, items + 1) if items % g == 0])
        if sched in ("serial_ascending", "descending_q"):
            opts["dispatch"] = "ring"
    elif sched != "auto" and rng.random() < 0.3:
        opts["dispatch"] = "ticket"
    if sched != "atomic_nondet" and rng.random() < 0.3:
        opts["dq_mode"] = rng.choice(["rmw", "atomic"])
    if rng.random() < 0.3:
        opts["grid"] = rng.choice([8, 16, 40, 64, 256])
    return (rng.choice([1, 2]), rng.choice([1, 2, 3]), S, D, causal, sched, opts)


CASES = [draw(random.Random(1000 + x)) for x in range(24)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}-{c[5]}")
def test_random_plan_matches_oracle(case):
    B, H, S, D, causal, sched, opts = case
    try:
        plan = da.detattn_bwd_plan(B, H, S, D, causal, sched, **opts)
    except da.DetAttnError:
        pytest.skip(f"plan not supported: {opts}")   # e.g. a ring wider than the grid
    say(f"[random] {case} plan {plan}")
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, 7 + S + D, causal)
    dq_r, dk_r, dv_r, _, _ = oref.attn_bwd(*cpu, 1.0 / math.sqrt(D), causal)
    ws = da.alloc_workspace(B, H, S, D)
    got = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                        workspace=ws, **opts)]
    assert da.detattn_device_status(ws) == 0
    for name, g, want in zip(("dq", "dk", "dv"), got, (dq_r, dk_r, dv_r)):
        e = rel_err(g.float().cpu().numpy(), want)
        assert e <= TOL, f"{name} rel err {e:.3e}"
    if plan["schedule"] != da.SCHEDULES["atomic_nondet"]:
        again = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, **opts)
        assert da.detattn_device_status(ws) == 0
        assert all(same_bits(a, b) for a, b in zip(got, again))
