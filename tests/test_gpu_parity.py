"""GPU parity of the HIP path against the fp64 oracle, and bitwise determinism.

Bar (for dQ, dK, dV separately): max|gpu - oracle| <= 2e-2 * max|oracle| on the
same bf16 inputs; every deterministic schedule is bit-identical across runs;
schedules that share an accumulation order agree bit for bit:
  * dQ: serial_ascending == descending_q (both add KV tiles in ascending order);
  * dK, dV: serial_ascending == atomic_nondet (both sweep Q tiles upward);
  * every output of a deterministic schedule is invariant under the grid size,
    the XCD placement and injected delays.
"""
import math

import numpy as np
import pytest
import torch

import deterministic_attention_backward_fa_amd as da
from oracle import ref as oref

from gpu_util import TOL, inputs, rel_err, same_bits, say

pytestmark = pytest.mark.gpu

SMALL = [
    # (B, H, S, D, causal, seed, options) -- oracle runs on the full tensors
    (1, 2, 256, 64, False, 101, {}),                                   # the 1x2x256x64 full-mask case
    (2, 3, 256, 64, True, 7, {}),
    (1, 2, 512, 64, True, 11, {}),                                     # 128x128 tiles, 4 KV tiles
    (1, 2, 512, 64, False, 12, {}),
    (1, 1, 512, 64, True, 13, {"block_q": 64, "block_kv": 128}),      # r = 2 at D = 64
    (1, 2, 512, 128, False, 14, {}),                                   # 64x128 tiles, r = 2
    (1, 2, 512, 128, True, 15, {}),
    (1, 2, 768, 128, True, 18, {}),                                    # 6 KV tiles: 3 symmetric pairs, r = 2
    (1, 2, 256, 128, False, 16, {"block_q": 64, "block_kv": 64}),     # the long-context tile shape
    (1, 2, 256, 128, True, 17, {"block_q": 64, "block_kv": 64}),
]


def plan_mode_name(plan):
    return {v: k for k, v in da.DQ_MODES.items()}[plan["dq_mode"]]


def schedules_for(causal):
    base = ["serial_ascending", "descending_q", "atomic_nondet"]
    return base + (["symmetric_shift"] if causal else ["shift"])


def _oracle(cpu, causal, scale):
    q, k, v, do = cpu
    return oref.attn_bwd(q, k, v, do, scale, causal)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_forward_matches_oracle(case):
    B, H, S, D, causal, seed, _ = case
    say(f"[fwd parity] {case}")
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    scale = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oref.attn_fwd(cpu[0], cpu[1], cpu[2], scale, causal)
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL
    assert np.max(np.abs(lse.cpu().numpy() - lse_ref)) <= 1e-3


@pytest.mark.parametrize("scale", [1.0, 0.0, -0.3])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_other_scales_match_oracle(scale, D, causal):
    # a positive scale takes the instance that finds the tile maximum on the raw
    # scores; zero and negative scales take the one that scales every score first
    B, H, S = 1, 2, 384
    say(f"[fwd scale] scale={scale} D={D} causal={causal}")
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, 19, causal, scale=scale)
    o_ref, lse_ref = oref.attn_fwd(cpu[0], cpu[1], cpu[2], scale, causal)
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL
    assert np.max(np.abs(lse.cpu().numpy() - lse_ref)) <= 1e-3


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_backward_matches_oracle_all_schedules(case):
    B, H, S, D, causal, seed, opts = case
    scale = 1.0 / math.sqrt(D)
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    dq_r, dk_r, dv_r, _, _ = _oracle(cpu, causal, scale)
    res = {}
    for sched in schedules_for(causal):
        say(f"[bwd parity] {case} {sched}")
        ws = da.alloc_workspace(B, H, S, D)
        dq, dk, dv = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws,
                                               **opts)
        assert da.detattn_device_status(ws) == 0
        for name, got, want in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
            e = rel_err(got.float().cpu().numpy(), want)
            assert e <= TOL, f"{sched} {name} rel err {e:.3e}"
        res[sched] = (dq, dk, dv)
    # the atomic reference both ways: device-scope atomics (ticket counter, the
    # default) and atomics in one XCD's L2 (rings of one XCD)
    say(f"[bwd parity] {case} atomic_nondet ring dispatch")
    ws = da.alloc_workspace(B, H, S, D)
    dq, dk, dv = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule="atomic_nondet",
                                           workspace=ws, dispatch="ring", **opts)
    assert da.detattn_device_status(ws) == 0
    for name, got, want in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        e = rel_err(got.float().cpu().numpy(), want)
        assert e <= TOL, f"atomic_nondet (ring) {name} rel err {e:.3e}"
    assert same_bits(res["atomic_nondet"][1], dk) and same_bits(res["atomic_nondet"][2], dv)
    # shared accumulation orders give identical bits
    assert same_bits(res["serial_ascending"][0], res["descending_q"][0])
    assert same_bits(res["serial_ascending"][1], res["atomic_nondet"][1])
    assert same_bits(res["serial_ascending"][2], res["atomic_nondet"][2])


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[6], SMALL[8]],
                         ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_bitwise_determinism_100_runs(case):
    B, H, S, D, causal, seed, opts = case
    _, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    for sched in [s for s in schedules_for(causal) if s != "atomic_nondet"]:
        say(f"[determinism x100] {case} {sched}")
        ws = da.alloc_workspace(B, H, S, D)
        first = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                             workspace=ws, **opts)]
        out = tuple(torch.empty_like(t) for t in first)
        for _ in range(99):
            da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out, **opts)
            for a, b in zip(first, out):
                assert same_bits(a, b), sched
        assert da.detattn_device_status(ws) == 0


@pytest.mark.parametrize("case", [SMALL[1], SMALL[3], SMALL[5], SMALL[6], SMALL[7]],
                         ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_invariance_grid_placement_delays(case):
    B, H, S, D, causal, seed, opts = case
    _, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    for sched in [s for s in schedules_for(causal) if s != "atomic_nondet"]:
        ws = da.alloc_workspace(B, H, S, D)
        say(f"[invariance] {case} {sched} baseline")
        base = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                            workspace=ws, **opts)]
        plan = da.detattn_bwd_plan(B, H, S, D, causal, sched, **opts)
        variants = [dict(debug_delay_seed=12345), dict(xcd_remap=False), dict(dq_mode="atomic"),
                    dict(dq_mode="rmw"), dict(cooperative_launch=True)]
        if sched in ("serial_ascending", "descending_q"):
            # static rings instead of the ticket counter: the same order (rank = KV tile), so the
            # same add mechanism gives the same bits
            variants += [dict(dispatch="ring"), dict(dispatch="ring", dq_mode=plan_mode_name(plan)),
                         dict(dispatch="ring", ring_size=1, grid=8)]
            n_kv = plan["n_kv"]
            if n_kv % 2 == 0 and n_kv >= 4:
                # two workgroups per ring, several rounds: descending hands out odd rounds
                # in reverse under a causal mask (snake order); the bits stay the same
                variants.append(dict(dispatch="ring", ring_size=2, dq_mode=plan_mode_name(plan)))
        ring = plan["ring"]
        if ring:
            variants.append(dict(grid=ring))           # a single ring at a time
            variants.append(dict(grid=ring * 2 + 8))   # uneven grid
        else:
            variants += [dict(grid=1), dict(grid=3), dict(grid=37)]
        for var in variants:
            say(f"[invariance] {case} {sched} {var}")
            got = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws,
                                            **opts, **var)
            assert da.detattn_device_status(ws) == 0
            # dK and dV never depend on the dQ mechanism or placement
            assert same_bits(base[1], got[1]) and same_bits(base[2], got[2]), (sched, var)
            vplan = da.detattn_bwd_plan(B, H, S, D, causal, sched, **opts, **var)
            if vplan["dq_mode"] == plan["dq_mode"]:
                assert same_bits(base[0], got[0]), (sched, var)
            else:
                # same order, another add mechanism (VALU add vs fp32 atomic): equal up to rounding of denormals
                assert rel_err(got[0].float().cpu().numpy(), base[0].float().cpu().numpy()) <= 1e-2


MISPLACE_CASES = [
    # (B, H, S, D, causal, seed, schedule): XCD-local rings by default
    (2, 16, 1024, 64, True, 81, "symmetric_shift"),
    (1, 32, 2048, 128, True, 82, "symmetric_shift"),
    (2, 16, 1024, 128, False, 83, "shift"),
    (2, 16, 2048, 128, False, 84, "descending_q"),
]


@pytest.mark.parametrize("case", MISPLACE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}-{c[6]}")
def test_wrong_placement_guess_changes_no_bit(case):
    """Rings of one XCD are formed from the XCD each workgroup reports. With
    the static guess shifted by one workgroup (debug_misplace), the registered
    placement differs from the guess for the workgroups, which drop their first
    loads and start over on their registered ring: the outputs are the same
    bits as with the right guess, and the call reports no error."""
    B, H, S, D, causal, seed, sched = case
    _, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    plan = da.detattn_bwd_plan(B, H, S, D, causal, sched)
    assert plan["ring"] > 0 and plan["dq_mode"] == da.DQ_MODES["xcd_local"], plan
    ws = da.alloc_workspace(B, H, S, D)
    say(f"[misplace] {case} plan {plan}")
    base = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                        workspace=ws)]
    for _ in range(3):
        got = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws,
                                        debug_misplace=True)
        assert da.detattn_device_status(ws) == 0
        assert all(same_bits(a_, b_) for a_, b_ in zip(base, got))


def test_plain_ring_launch_refuses_a_grid_beyond_residency():
    """Ring dispatch launched plainly needs the whole grid resident at once: an
    explicit grid larger than compute units x occupancy is refused before any
    kernel runs (the outputs keep what the caller put there)."""
    B, H, S, D = 4, 32, 1024, 128
    _, (q, k, v, do, o, lse) = inputs(B, H, S, D, 71, True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = da.detattn_bwd_plan(B, H, S, D, True, "symmetric_shift", grid=4 * cus)
    assert plan["ring"] > 0 and plan["grid"] > cus and plan["cooperative"] == 0
    ws = da.alloc_workspace(B, H, S, D)
    out = tuple(torch.full_like(q, 7.0) for _ in range(3))
    say(f"[residency] plan {plan}")
    with pytest.raises(da.DetAttnError) as ei:
        da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=True, schedule="symmetric_shift", workspace=ws,
                                  out=out, grid=4 * cus)
    assert "UNSUPPORTED" in str(ei.value)
    torch.cuda.synchronize()
    assert all(bool(torch.all(t == 7.0)) for t in out)
    # the default grid fits, plainly and cooperatively, with the same bits
    a = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=True, schedule="symmetric_shift",
                                                      workspace=ws)]
    b = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=True, schedule="symmetric_shift", workspace=ws,
                                  cooperative_launch=True)
    assert da.detattn_device_status(ws) == 0
    assert all(same_bits(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("dispatch", ["ticket", "ring"])
def test_timeout_path_reports_and_exits(dispatch):
    """Withhold one workgroup's first dQ signal: its successor's bounded wait
    expires, the error word is set and every kernel still exits."""
    B, H, S, D = 1, 1, 256, 64
    _, (q, k, v, do, o, lse) = inputs(B, H, S, D, 3, False)
    ws = da.alloc_workspace(B, H, S, D)
    say(f"[timeout path] serial_ascending ({dispatch} dispatch), item 0 withholds its first signal")
    da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=False, schedule="serial_ascending", workspace=ws,
                              debug_skip_signal=1, timeout_us=2000, dispatch=dispatch)
    # the status is sticky: a later successful call on the workspace does not hide the failure
    da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=False, schedule="serial_ascending", workspace=ws,
                              dispatch=dispatch)
    assert da.detattn_device_status(ws) == 5
    # reading the status clears it; a normal call leaves it clean
    assert da.detattn_device_status(ws) == 0
    da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=False, schedule="serial_ascending", workspace=ws,
                              dispatch=dispatch)
    assert da.detattn_device_status(ws) == 0
    # the binding's check raises on the failing call itself
    say(f"[timeout path] check=True raises")
    with pytest.raises(da.DetAttnError):
        da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=False, schedule="serial_ascending", workspace=ws,
                                  debug_skip_signal=1, timeout_us=2000, dispatch=dispatch, check=True)
    assert da.detattn_device_status(ws) == 0


RING_CASES = [
    # (B, H, S, D, causal, seed, options, ring sizes): heads with more items than ring workgroups
    (1, 2, 512, 64, False, 21, {"block_q": 64, "block_kv": 64}, (1, 2, 4)),   # shift, 8 items
    (1, 2, 512, 128, True, 22, {"block_q": 64, "block_kv": 64}, (1, 2)),      # symmetric, 4 items
    (1, 2, 1024, 128, True, 23, {}, (1, 2)),                                  # symmetric, r = 2
    (1, 1, 1024, 128, False, 24, {}, (2, 4)),                                 # shift, r = 2
    (1, 2, 1536, 128, True, 25, {}, (1, 3)),                                  # symmetric, 6 pairs, r = 2
]


@pytest.mark.parametrize("case", RING_CASES, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_ring_rounds_match_oracle_and_repeat(case):
    """Rings smaller than the item count (items taken in rounds): oracle parity,
    repeat and placement invariance at a fixed ring size, and dK/dV independent
    of the ring size (they never depend on the dQ order)."""
    B, H, S, D, causal, seed, opts, rings = case
    sched = "symmetric_shift" if causal else "shift"
    scale = 1.0 / math.sqrt(D)
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    dq_r, dk_r, dv_r, _, _ = _oracle(cpu, causal, scale)
    ws = da.alloc_workspace(B, H, S, D)
    first_dkdv = None
    for G in rings:
        plan = da.detattn_bwd_plan(B, H, S, D, causal, sched, ring_size=G, **opts)
        assert plan["ring"] == G
        say(f"[ring rounds] {case[:6]} {sched} ring {G} plan {plan}")
        base = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                            workspace=ws, ring_size=G, **opts)]
        assert da.detattn_device_status(ws) == 0
        for name, got, want in (("dq", base[0], dq_r), ("dk", base[1], dk_r), ("dv", base[2], dv_r)):
            e = rel_err(got.float().cpu().numpy(), want)
            assert e <= TOL, f"ring {G} {name} rel err {e:.3e}"
        if first_dkdv is None:
            first_dkdv = base[1:]
        assert same_bits(first_dkdv[0], base[1]) and same_bits(first_dkdv[1], base[2])
        out = tuple(torch.empty_like(t) for t in base)
        for _ in range(9):
            da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out,
                                      ring_size=G, **opts)
            assert all(same_bits(a, b) for a, b in zip(base, out)), f"ring {G} repeat"
        for var in (dict(debug_delay_seed=777), dict(grid=G * 2 + 8), dict(grid=G)):
            say(f"[ring rounds] ring {G} {var}")
            got = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws,
                                            ring_size=G, **opts, **var)
            assert da.detattn_device_status(ws) == 0
            vplan = da.detattn_bwd_plan(B, H, S, D, causal, sched, ring_size=G, **opts, **var)
            assert same_bits(base[1], got[1]) and same_bits(base[2], got[2]), var
            if vplan["dq_mode"] == plan["dq_mode"]:
                assert same_bits(base[0], got[0]), var
            else:
                assert rel_err(got[0].float().cpu().numpy(), base[0].float().cpu().numpy()) <= 1e-2


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_gradient_identities_on_gpu_output(case):
    """Rows of dS sum to zero, so the keys' dK sum to zero; rows of P sum to one,
    so the keys' dV sum to the queries' dO. The bf16 outputs meet both up to
    their rounding (relative 1e-2 of the summed magnitudes)."""
    B, H, S, D, causal, seed, opts = case
    _, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    for sched in schedules_for(causal):
        say(f"[identities] {case} {sched}")
        ws = da.alloc_workspace(B, H, S, D)
        dq, dk, dv = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws,
                                               **opts)
        assert da.detattn_device_status(ws) == 0
        dk64, dv64, do64 = (t.double().cpu() for t in (dk, dv, do))
        sk = dk64.sum(dim=2).abs()
        assert torch.all(sk <= 1e-2 * dk64.abs().sum(dim=2) + 1e-6), sched
        sv = (dv64.sum(dim=2) - do64.sum(dim=2)).abs()
        assert torch.all(sv <= 1e-2 * dv64.abs().sum(dim=2) + 1e-6), sched


TRACE_CASES = [
    # (B, H, S, D, causal, seed, options): two small shapes per mask, both head dimensions
    (1, 2, 512, 64, False, 31, {}),
    (1, 2, 512, 128, False, 32, {}),
    (1, 2, 512, 64, True, 33, {}),
    (1, 2, 1024, 128, True, 34, {}),
]


@pytest.mark.parametrize("case", TRACE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}{'c' if c[4] else 'f'}")
def test_traced_instances_match_oracle_and_untraced_bits(case):
    """The phase-traced kernel instances (their own translation units) compute
    the same thing: oracle parity at the same bar, and every output bit-equal to
    the untraced instance of the same plan; the trace records are well formed."""
    B, H, S, D, causal, seed, opts = case
    scale = 1.0 / math.sqrt(D)
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
    dq_r, dk_r, dv_r, _, _ = _oracle(cpu, causal, scale)
    for sched in schedules_for(causal):
        if sched == "atomic_nondet":
            continue
        plan = da.detattn_bwd_plan(B, H, S, D, causal, sched, **opts)
        recs = 64
        trace = torch.zeros(plan["grid"] * recs * 2, dtype=torch.int64, device="cuda")
        ws = da.alloc_workspace(B, H, S, D)
        say(f"[traced] {case[:5]} {sched} plan {plan}")
        base = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                            workspace=ws, **opts)]
        got = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws,
                                        trace=trace, trace_records=recs, **opts)
        assert da.detattn_device_status(ws) == 0
        for name, g, want in (("dq", got[0], dq_r), ("dk", got[1], dk_r), ("dv", got[2], dv_r)):
            e = rel_err(g.float().cpu().numpy(), want)
            assert e <= TOL, f"traced {sched} {name} rel err {e:.3e}"
        assert all(same_bits(a, b) for a, b in zip(base, got)), f"traced {sched} differs from untraced"
        t = trace.view(plan["grid"], recs, 2).cpu()
        used = t[:, :, 0] != 0
        assert used.any()
        phases = (t[:, :, 1] & 0xFF)[used]
        assert int(phases.max()) <= 9
        # timestamps never decrease within a workgroup's records
        for w in range(plan["grid"]):
            ts = t[w, :, 0][used[w]]
            assert torch.all(ts[1:] >= ts[:-1]), (sched, w)


PAIR_CASES = [
    # (B, H, S, D, seed, ring sizes): causal, 64 x 64 tiles, D = 64
    (1, 2, 512, 64, 61, (0, 2)),
    (2, 3, 1024, 64, 62, (0, 4)),
    (1, 1, 2048, 64, 63, (0,)),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}D{c[3]}")
def test_resident_pair_symmetric_shift_equals_sequential(case):
    """Symmetric shift with both columns of a pair item resident in registers
    (the register-pressure alternative the pages discuss) visits the same tiles
    in the same order as the one-column-at-a-time form: every output bit is the
    same, it meets the oracle, and it repeats bit for bit."""
    B, H, S, D, seed, rings = case
    opts = dict(block_q=64, block_kv=64)
    scale = 1.0 / math.sqrt(D)
    cpu, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, True)
    dq_r, dk_r, dv_r, _, _ = _oracle(cpu, True, scale)
    ws = da.alloc_workspace(B, H, S, D)
    for G in rings:
        ring = dict(ring_size=G) if G else {}
        plan = da.detattn_bwd_plan(B, H, S, D, True, "symmetric_shift", pair_columns=True, **opts, **ring)
        assert plan["pair_columns"] == 1
        say(f"[resident pair] {case[:4]} ring {G or 'default'} plan {plan}")
        seq = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=True, schedule="symmetric_shift",
                                                            workspace=ws, **opts, **ring)]
        pair = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=True,
                                                             schedule="symmetric_shift", workspace=ws,
                                                             pair_columns=True, **opts, **ring)]
        assert da.detattn_device_status(ws) == 0
        assert all(same_bits(a_, b_) for a_, b_ in zip(seq, pair))
        for name, got, want in (("dq", pair[0], dq_r), ("dk", pair[1], dk_r), ("dv", pair[2], dv_r)):
            e = rel_err(got.float().cpu().numpy(), want)
            assert e <= TOL, f"resident pair {name} rel err {e:.3e}"
        for _ in range(9):
            again = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=True, schedule="symmetric_shift", workspace=ws,
                                              pair_columns=True, **opts, **ring)
            assert all(same_bits(a_, b_) for a_, b_ in zip(pair, again))
        assert da.detattn_device_status(ws) == 0
