"""Full-size GPU checks in the launch configuration the benchmark times.

For every workload shape below, every valid schedule runs with the library's
default plan (tiles, grid, rings, dQ mode). The fp64 oracle computes sampled
outputs one by one on three heads (the first, a middle and the last; two at
64k tokens): dQ at sampled query rows, dK and dV at sampled key rows (32 random
positions each, plus the first and last and the positions around 64- and
128-row tile edges and the sequence's midpoint, where symmetric shift's
rectangle starts), plus every row's log-sum-exp. The bar is
the same as for the small cases, max|gpu - oracle| <= 2e-2 * max|oracle| over
the sampled values, and the bitwise relations between schedules that share an
accumulation order hold at full size. Every deterministic schedule of the
workload shapes repeats 100 times (2 at 64k tokens) with identical bits and a
clean device status after every call; the SHA-256 of each schedule's outputs
is printed.
"""
import hashlib
import math

import numpy as np
import pytest
import torch

import deterministic_attention_backward_fa_amd as da
from deterministic_attention_backward_fa_amd.synth import make_qkvdo, sample_indices
from oracle import ref as oref

from gpu_util import TOL, rel_err, same_bits, say

pytestmark = pytest.mark.gpu

CONFIGS = {
    # name: (B, H, S, D, causal, seed, runs for the determinism check, options)
    "causal_b4_h16_s2048_d64": (4, 16, 2048, 64, True, 102, 100, {}),
    "full_b2_h32_s4096_d128": (2, 32, 4096, 128, False, 103, 100, {}),
    "causal_b1_h32_s8192_d128": (1, 32, 8192, 128, True, 104, 100, {}),
    # the long-context workload with its stated 64-row KV tile, then with the library's default tile
    "full_b1_h16_s16384_d128_kv64": (1, 16, 16384, 128, False, 105, 100, {"block_q": 64, "block_kv": 64}),
    "causal_b1_h16_s16384_d128_kv64": (1, 16, 16384, 128, True, 105, 100, {"block_q": 64, "block_kv": 64}),
    "full_b1_h16_s16384_d128": (1, 16, 16384, 128, False, 105, 100, {}),
    "causal_b1_h16_s16384_d128": (1, 16, 16384, 128, True, 105, 100, {}),
    # the longest context here: 64k tokens (offsets and flag counts at their largest in this suite)
    "full_b1_h4_s65536_d128": (1, 4, 65536, 128, False, 106, 2, {}),
    "causal_b1_h4_s65536_d128": (1, 4, 65536, 128, True, 106, 2, {}),
}


def schedules_for(causal):
    return ["serial_ascending", "descending_q", "symmetric_shift" if causal else "shift", "atomic_nondet"]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_fullsize_sampled_parity_and_determinism(name):
    B, H, S, D, causal, seed, runs, opts = CONFIGS[name]
    scale = 1.0 / math.sqrt(D)
    say(f"[fullsize] {name}: inputs")
    cpu = make_qkvdo(B, H, S, D, seed)
    q, k, v, do = (t.cuda() for t in cpu)
    o, lse = da.detattn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    edges = {63, 64, 127, 128, S // 2 - 1, S // 2, S - 65, S - 64}
    rows = sorted(set(sample_indices(S, 32, seed)) | {x for x in edges if 0 <= x < S})
    cols = sorted(set(sample_indices(S, 32, seed + 1)) | {x for x in edges if 0 <= x < S})
    heads = [(0, 0), (B // 2, H // 2), (B - 1, H - 1)] if S <= 16384 else [(0, 0), (B - 1, H - 1)]
    refs = {}
    for (b, h) in heads:
        say(f"[fullsize] {name}: oracle head ({b},{h})")
        refs[(b, h)] = oref.attn_bwd_sampled(cpu[0][b, h], cpu[1][b, h], cpu[2][b, h], cpu[3][b, h], scale, causal,
                                             rows, cols)
        # forward statistics of the library against the oracle's, every row
        assert np.max(np.abs(lse[b, h].cpu().numpy() - refs[(b, h)][3])) <= 1e-3
    outs = {}
    for sched in schedules_for(causal):
        say(f"[fullsize] {name}: {sched} plan {da.detattn_bwd_plan(B, H, S, D, causal, sched, **opts)}")
        ws = da.alloc_workspace(B, H, S, D)
        first = [t.clone() for t in da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched,
                                                             workspace=ws, **opts)]
        assert da.detattn_device_status(ws) == 0
        for (b, h) in heads:
            rdq, rdk, rdv, _, _ = refs[(b, h)]
            for label, got, want in (("dq", first[0][b, h, rows], rdq), ("dk", first[1][b, h, cols], rdk),
                                     ("dv", first[2][b, h, cols], rdv)):
                e = rel_err(got.float().cpu().numpy(), want)
                assert e <= TOL, f"{name} {sched} head ({b},{h}) {label}: rel err {e:.3e}"
        if sched != "atomic_nondet":
            digest = hashlib.sha256()
            for t in first:
                digest.update(t.view(torch.int16).cpu().numpy().tobytes())
            say(f"[fullsize] {name}: {sched} sha256(dq|dk|dv) {digest.hexdigest()}")
            out = tuple(torch.empty_like(t) for t in first)
            for run in range(runs - 1):
                da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=sched, workspace=ws, out=out,
                                          **opts)
                assert da.detattn_device_status(ws) == 0, f"{name} {sched} run {run + 2}: device status"
                for a, b_ in zip(first, out):
                    assert same_bits(a, b_), f"{name} {sched} run {run + 2} not bit-identical to run 1"
            say(f"[fullsize] {name}: {sched} {runs} runs bit-identical")
        outs[sched] = first
    if not opts:
        # the automatic choice is the measured-fastest deterministic schedule: same plan, same bits
        auto = da.detattn_bwd_plan(B, H, S, D, causal, "auto")
        name_auto = da.SCHEDULE_NAMES[auto["schedule"]]
        got = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule="auto")
        assert all(same_bits(a, b_) for a, b_ in zip(outs[name_auto], got)), name_auto
    assert same_bits(outs["serial_ascending"][0], outs["descending_q"][0])
    assert same_bits(outs["serial_ascending"][1], outs["atomic_nondet"][1])
    assert same_bits(outs["serial_ascending"][2], outs["atomic_nondet"][2])
