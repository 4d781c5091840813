"""Pins of the oracle's chunked-prefill attention.

A chunk of C new tokens ("PyTorch LLM Serving Engine", What is implemented:
configurable prefill chunks) is attended row by row at positions
L - C .. L - 1.  Pinned by: a chunk covering a whole sequence equals torch's
causal scaled_dot_product_attention (fp64, CPU) on the generated K/V; each
chunk row equals a decode over the matching prefix (decode is pinned in
test_oracle_attention); splitting a chunk changes nothing; window limits."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle.cases import build_cache, expected_outputs, to_numpy


def _prefill(seq_lens, new_lens, hq=8, hkv=2, d=64, window=0, seed=51, dtype="bf16"):
    return workloads.make_case("prefill", seed, seq_lens, new_lens, hq, hkv, d, in_dtype=dtype,
                               window=window, kind="prefill")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_whole_sequence_chunk_equals_causal_sdpa(dtype):
    case = _prefill([37, 80, 16], [37, 80, 16], dtype=dtype)
    got = expected_outputs(case)
    cu = case.cu_q_lens
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        q = case.q_seq(s).double().permute(1, 0, 2).unsqueeze(0)
        k = case.kv("k", s, 0, L).double().permute(1, 0, 2).unsqueeze(0)
        v = case.kv("v", s, 0, L).double().permute(1, 0, 2).unsqueeze(0)
        ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=float(case.softmax_scale),
                                             enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 24])
def test_each_chunk_row_equals_decode_over_its_prefix(window):
    case = _prefill([70, 33], [20, 33], window=window)
    cache = build_cache(case)
    got = expected_outputs(case, cache=cache)
    q = to_numpy(case.q())
    cu = case.cu_q_lens
    for s in range(case.num_seqs):
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        for i in range(C):
            row = cu[s] + i
            ref = oracle.decode(cache, q[row:row + 1], "bf16", np.array([L - C + i + 1], np.int32),
                                case.block_tables[s:s + 1], case.softmax_scale, window)
            assert np.array_equal(got[row], ref[0])


def test_one_row_chunk_is_decode():
    case = _prefill([45, 3, 18], [1, 1, 1])
    cache = build_cache(case)
    a = expected_outputs(case, cache=cache)
    b = oracle.decode(cache, to_numpy(case.q()), "bf16", case.seq_lens, case.block_tables,
                      case.softmax_scale)
    assert np.array_equal(a, b)


def test_splitting_a_chunk_changes_nothing():
    whole = _prefill([300], [256], window=100)
    cache = build_cache(whole)
    q = to_numpy(whole.q())
    ref = expected_outputs(whole, cache=cache)
    first = oracle.attention(cache, q[:128], "bf16", [0, 128], [172], whole.block_tables,
                             whole.softmax_scale, 100)
    second = oracle.attention(cache, q[128:], "bf16", [0, 128], [300], whole.block_tables,
                              whole.softmax_scale, 100)
    assert np.array_equal(np.concatenate([first, second]), ref)


def test_window_limits():
    base = dict(seq_lens=[50, 21], new_lens=[10, 21])
    one = _prefill(**base, window=1)
    out = expected_outputs(one)
    cu = one.cu_q_lens
    for s in range(2):
        L, C = int(one.seq_lens[s]), int(one.new_lens[s])
        v = one.kv("v", s, L - C, L).double().repeat_interleave(one.group, dim=1).numpy()
        assert np.array_equal(out[cu[s]:cu[s + 1]], v)
    assert np.array_equal(expected_outputs(_prefill(**base, window=0)),
                          expected_outputs(_prefill(**base, window=50)))
    assert not np.array_equal(expected_outputs(_prefill(**base, window=0)),
                              expected_outputs(_prefill(**base, window=49)))


def test_weights_sum_to_one_per_row():
    case = _prefill([40, 100], [40, 30], window=33)
    out, w = expected_outputs(case, weights=True)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert torch.count_nonzero(torch.from_numpy(w[0, 0])) == 1      # the first row sees only itself
