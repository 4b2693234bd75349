"""Helpers shared by the GPU tests: seeded inputs on the device and error metrics."""
import sys

import numpy as np
import torch

import deterministic_attention_backward_fa_amd as da
from deterministic_attention_backward_fa_amd.synth import make_qkvdo

TOL = 2e-2  # max|gpu - ref| <= TOL * max|ref| per tensor (bf16 inputs, fp32 accumulation)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(B, H, S, D, seed, causal, scale=None):
    """bf16 q, k, v, dO on the GPU plus O and LSE from the library's forward."""
    q, k, v, do = make_qkvdo(B, H, S, D, seed)
    dev = [t.cuda() for t in (q, k, v, do)]
    o, lse = da.detattn_fwd(dev[0], dev[1], dev[2], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, do), dev + [o, lse]


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (m if m > 0 else 1.0))


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def same_bits(a, b):
    return torch.equal(bits(a), bits(b))
