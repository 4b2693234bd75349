"""The entry point that allocates nothing (attn_bwd_deterministic_noalloc),
called through the C ABI: its results equal those of attn_bwd_deterministic
with a caller workspace (the same kernels, plan and order: bit for bit for the
ordered schedules, within the parity bar for the atomic one), over two calls in
a row with the second on a smaller shape; the scratch's status word reads clean;
a shape beyond the fixed scratch is refused before any launch."""
import ctypes

import pytest
import torch

import deterministic_attention_backward_fa_amd as da

from gpu_util import inputs, rel_err, same_bits, say

pytestmark = pytest.mark.gpu

CALLS = [
    # (B, H, S, D, causal, seed, schedule): the second call is smaller than the first
    (1, 8, 2048, 128, True, 41, "symmetric_shift"),
    (1, 2, 512, 64, False, 42, "shift"),
]


def test_noalloc_matches_workspace_entry_point_twice():
    for (B, H, S, D, causal, seed, sched) in CALLS:
        _, (q, k, v, do, o, lse) = inputs(B, H, S, D, seed, causal)
        for s in (sched, "descending_q", "atomic_nondet"):
            say(f"[no-alloc] B{B} H{H} S{S} D{D} {'causal' if causal else 'full'} {s}")
            ws = da.alloc_workspace(B, H, S, D)
            want = da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=s, workspace=ws)
            assert da.detattn_device_status(ws) == 0
            out = (torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0))
            got = da.attn_bwd_deterministic_noalloc(q, k, v, o, do, lse, causal=causal, schedule=s, out=out)
            assert da.detattn_device_status(None) == 0
            if s == "atomic_nondet":
                assert same_bits(want[1], got[1]) and same_bits(want[2], got[2])
                assert rel_err(got[0].float().cpu().numpy(), want[0].float().cpu().numpy()) <= 1e-2
            else:
                for a, b in zip(want, got):
                    assert same_bits(a, b), s


def test_noalloc_refuses_shapes_beyond_its_scratch():
    L = da.lib()
    p = ctypes.c_void_p(0x10000)
    big = da.Shape(1, 64, 8192, 128, 0.088)    # 2^26 elements: a 256 MiB accumulator
    assert da.detattn_bwd_workspace_bytes(1, 64, 8192, 128) > da.NOALLOC_SCRATCH_BYTES
    assert L.attn_bwd_deterministic_noalloc(p, p, p, p, p, p, p, p, p, big, 1, 3, None) == 7
