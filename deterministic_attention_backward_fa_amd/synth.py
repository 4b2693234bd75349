"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the attention arithmetic. Recipe: a CPU ``torch.Generator`` seeded with
``seed`` draws q, k, v and dO in that order from N(0, 1) in fp32 (the pages
benchmark on random bf16 inputs), then each is rounded to bf16 with
round-to-nearest-even by ``Tensor.to``.
"""
import torch


def make_qkvdo(B, H, S, D, seed, dtype=torch.bfloat16):
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for _ in range(4):
        t = torch.randn((B, H, S, D), generator=g, dtype=torch.float32)
        out.append(t.to(dtype) if dtype != torch.float32 else t)
    return tuple(out)


def sample_indices(S, count, seed):
    """Distinct sorted positions in [0, S) that always include the first and last ones."""
    g = torch.Generator("cpu").manual_seed(int(seed) + 7919)
    count = min(count, S)
    perm = torch.randperm(S, generator=g)[: max(count - 2, 0)].tolist()
    idx = sorted(set(perm) | {0, S - 1})
    return idx[:count] if len(idx) > count else idx
