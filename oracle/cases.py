"""Run the oracle on a seeded workload (test infrastructure only).

Takes a ``workloads.PagedCase`` -- inputs only -- and computes with the oracle
what the GPU library must reproduce: the expected pool bytes after the cache
write of every token, and the expected attention outputs.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Cache, attention, decode

__all__ = ["to_numpy", "build_cache", "expected_outputs"]


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a generated tensor; bf16 as uint16 bit patterns."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def build_cache(case, kv_dtype: str | None = None, include_new: bool = True, device="cpu") -> Cache:
    """Poisoned pool, then every context token (and the step's new tokens)
    written through the reference cache write, sequence by sequence.  The
    inputs are generated on ``device`` (the generator is bit-identical on
    CPU and GPU) and copied to the host; the oracle itself runs on the host."""
    cache = Cache(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim,
                  kv_dtype or case.kv_dtype)
    for s in range(case.num_seqs):
        p0, p1 = case.context_range(s)
        if include_new:
            p1 = int(case.seq_lens[s])
        if p1 <= p0:
            continue
        k = to_numpy(case.kv("k", s, p0, p1, device))
        v = to_numpy(case.kv("v", s, p0, p1, device))
        cache.write(k, v, case.in_dtype, case.slots(s, p0, p1))
    return cache


def expected_outputs(case, cache: Cache | None = None, kv_dtype: str | None = None,
                     weights: bool = False):
    """Oracle attention output for every query row of the step: [rows][Hq][D] fp64."""
    if cache is None:
        cache = build_cache(case, kv_dtype)
    q = to_numpy(case.q())
    if case.kind == "decode":
        return decode(cache, q, case.in_dtype, case.seq_lens, case.block_tables,
                      case.softmax_scale, case.window, weights=weights)
    return attention(cache, q, case.in_dtype, case.cu_q_lens, case.seq_lens, case.block_tables,
                     case.softmax_scale, case.window, weights=weights)
