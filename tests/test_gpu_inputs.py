"""The seeded generator gives bit-identical inputs on the CPU and the GPU.

The oracle's inputs for full-size cases are generated on the GPU by the
generator (integer hashing only) and copied to the host; this pins that
they equal the CPU generation bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from oracle.cases import to_numpy

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("make", [workloads.tiny_fp32_decode, workloads.int8_decode, workloads.llama_decode])
def test_generated_values_match_across_devices(make):
    case = make()
    dev = torch.device("cuda", 0)
    for s in (0, case.num_seqs - 1):
        L = int(case.seq_lens[s])
        for which in ("k", "v"):
            a = to_numpy(case.kv(which, s, 0, L))
            b = to_numpy(case.kv(which, s, 0, L, dev))
            assert np.array_equal(a, b)
    assert np.array_equal(to_numpy(case.q()), to_numpy(case.q(dev)))


def test_hash_words_match_across_devices():
    idx = torch.arange(0, 1 << 20, dtype=torch.int64) * 977 + (1 << 33)
    a = workloads.hash_u32(5, 2, idx)
    b = workloads.hash_u32(5, 2, idx.cuda()).cpu()
    assert torch.equal(a, b)
