"""Pins of the oracle's decode attention.

The method ("PyTorch LLM Serving Engine", Loading and What is implemented)
walks a block table with a stable online softmax; that reaches plain
softmax attention, so the oracle must equal it.  Pinned here by:
  * torch's scaled_dot_product_attention in fp64 on the CPU (the dense
    uncached path that page names) fed with the generated K/V directly,
    so the cache write, the block table and the gather are all covered;
  * grouped-query sharing against explicitly repeated KV heads ("MicroGen",
    Key Features: repeat_kv);
  * invariants (block permutation, weights summing to 1) and closed forms
    (one- and two-token contexts, zero scale, window of one, huge scores).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle.cases import build_cache, expected_outputs, to_numpy


def _sdpa_decode(case, window=None, repeat=False):
    """Dense fp64 attention of each sequence's query over its generated K/V."""
    window = case.window if window is None else window
    outs = []
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        lo = max(0, L - window) if window > 0 else 0
        q = case.q_seq(s).double().permute(1, 0, 2).unsqueeze(0)            # [1, Hq, 1, D]
        k = case.kv("k", s, lo, L).double().permute(1, 0, 2).unsqueeze(0)   # [1, Hkv, L', D]
        v = case.kv("v", s, lo, L).double().permute(1, 0, 2).unsqueeze(0)
        if repeat:
            k = k.repeat_interleave(case.group, dim=1)
            v = v.repeat_interleave(case.group, dim=1)
        o = F.scaled_dot_product_attention(q, k, v, scale=float(case.softmax_scale),
                                           enable_gqa=not repeat)
        outs.append(o[0].permute(1, 0, 2))
    return torch.cat(outs).numpy()


CASES = [
    dict(seq_lens=[7, 16, 33, 50], hq=4, hkv=2, d=64, dtype="f32"),
    dict(seq_lens=[1, 2, 15, 17, 100, 257], hq=12, hkv=2, d=128, dtype="bf16"),
    dict(seq_lens=[64, 300], hq=8, hkv=8, d=64, dtype="bf16"),
    dict(seq_lens=[90, 31], hq=6, hkv=1, d=128, dtype="f32"),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"G{c['hq'] // c['hkv']}-D{c['d']}-{c['dtype']}")
@pytest.mark.parametrize("window", [0, 20])
def test_decode_equals_dense_sdpa(c, window):
    case = workloads.make_case("pin", 31, c["seq_lens"], [1] * len(c["seq_lens"]), c["hq"], c["hkv"],
                               c["d"], in_dtype=c["dtype"], window=window)
    got = expected_outputs(case)
    ref = _sdpa_decode(case)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got, _sdpa_decode(case, repeat=True), rtol=0, atol=1e-12)


def test_block_permutation_leaves_output_bit_identical():
    case = workloads.make_case("perm", 32, [5, 40, 129], [1, 1, 1], 8, 2, 128)
    compact = case.subset(range(case.num_seqs))            # same values, contiguous blocks
    assert not np.array_equal(case.block_tables[:, :2], compact.block_tables[:, :2])
    assert np.array_equal(expected_outputs(case), expected_outputs(compact))


def test_weights_sum_to_one_and_vanish_outside_the_visible_keys():
    for window in (0, 7):
        case = workloads.make_case("w", 33, [1, 9, 48, 77], [1] * 4, 4, 2, 64, window=window)
        out, w = expected_outputs(case, weights=True)
        assert np.isfinite(out).all()
        for s in range(case.num_seqs):
            L = int(case.seq_lens[s])
            lo = max(0, L - window) if window else 0
            np.testing.assert_allclose(w[s].sum(-1), 1.0, rtol=0, atol=1e-12)
            assert (w[s][:, :lo] == 0).all() and (w[s][:, L:] == 0).all()
            assert (w[s][:, lo:L] > 0).all()


def test_one_token_context_returns_that_value():
    case = workloads.make_case("one", 34, [1, 1], [1, 1], 4, 2, 64, in_dtype="bf16")
    out = expected_outputs(case)
    for s in range(2):
        v = case.kv("v", s, 0, 1).double()[0]             # [Hkv][D]
        assert np.array_equal(out[s], v.repeat_interleave(2, dim=0).numpy())


def test_two_token_context_by_hand():
    case = workloads.make_case("two", 35, [2], [1], 2, 1, 64, in_dtype="f32", softmax_scale=0.125)
    out = expected_outputs(case)
    q = case.q().double()[0]              # [2][D]
    k = case.kv("k", 0, 0, 2).double()[:, 0]
    v = case.kv("v", 0, 0, 2).double()[:, 0]
    for h in range(2):
        s0, s1 = 0.125 * float(q[h] @ k[0]), 0.125 * float(q[h] @ k[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))     # logistic form of a two-way softmax
        ref = w0 * v[0] + (1.0 - w0) * v[1]
        np.testing.assert_allclose(out[0, h], ref.numpy(), rtol=0, atol=1e-14)


def test_zero_scale_averages_the_visible_values():
    for window in (0, 5):
        case = workloads.make_case("zero", 36, [3, 21], [1, 1], 4, 2, 64, softmax_scale=0.0,
                                   window=window)
        out = expected_outputs(case)
        for s in range(2):
            L = int(case.seq_lens[s])
            lo = max(0, L - window) if window else 0
            mean = case.kv("v", s, lo, L).double().mean(0).repeat_interleave(2, dim=0).numpy()
            np.testing.assert_allclose(out[s], mean, rtol=0, atol=1e-14)


def test_window_of_one_returns_the_current_value_and_wide_window_is_no_window():
    base = dict(seq_lens=[9, 40], new_lens=[1, 1], num_q_heads=4, num_kv_heads=2, head_dim=64)
    one = workloads.make_case("w1", 37, **base, window=1)
    out = expected_outputs(one)
    for s in range(2):
        L = int(one.seq_lens[s])
        v = one.kv("v", s, L - 1, L).double()[0].repeat_interleave(2, dim=0).numpy()
        assert np.array_equal(out[s], v)
    none = workloads.make_case("w0", 37, **base, window=0)
    wide = workloads.make_case("w40", 37, **base, window=40)
    narrow = workloads.make_case("w39", 37, **base, window=39)
    assert np.array_equal(expected_outputs(none), expected_outputs(wide))
    assert not np.array_equal(expected_outputs(none)[1], expected_outputs(narrow)[1])


def test_huge_scores_stay_finite_and_pick_the_best_key():
    case = workloads.make_case("big", 38, [50], [1], 2, 1, 64, in_dtype="f32", softmax_scale=1e4)
    out = expected_outputs(case)
    assert np.isfinite(out).all()
    q = case.q().double()[0]
    k = case.kv("k", 0, 0, 50).double()[:, 0]
    v = case.kv("v", 0, 0, 50).double()[:, 0]
    for h in range(2):
        best = int(torch.argmax(k @ q[h]))
        np.testing.assert_allclose(out[0, h], v[best].numpy(), rtol=0, atol=1e-12)


def test_grouped_heads_match_explicitly_repeated_kv_heads():
    g = workloads.make_case("gqa", 39, [23, 70], [1, 1], 6, 2, 64)
    cache = build_cache(g)
    # the same K/V, each KV head copied G=3 times as its own head, in an MHA cache
    rep = oracle.Cache(g.num_blocks, 16, 6, 64, "bf16")
    rep.k[:] = np.repeat(cache.k, 3, axis=1)
    rep.v[:] = np.repeat(cache.v, 3, axis=1)
    q = to_numpy(g.q())
    a = oracle.decode(cache, q, "bf16", g.seq_lens, g.block_tables, g.softmax_scale)
    b = oracle.decode(rep, q, "bf16", g.seq_lens, g.block_tables, g.softmax_scale)
    assert np.array_equal(a, b)


def test_heads_of_a_group_with_equal_queries_agree():
    case = workloads.make_case("eqq", 40, [33], [1], 4, 1, 64)
    cache = build_cache(case)
    q = to_numpy(case.q())
    q[:, 1:] = q[:, :1]
    out = oracle.decode(cache, q, "bf16", case.seq_lens, case.block_tables, case.softmax_scale)
    for h in range(1, 4):
        assert np.array_equal(out[0, h], out[0, 0])


def test_empty_context_gives_zero_row():
    case = workloads.make_case("empty", 41, [0, 5], [1, 1], 4, 2, 64)
    cache = build_cache(case, include_new=False)
    cache2 = build_cache(case)
    out = oracle.decode(cache2, to_numpy(case.q()), "bf16", case.seq_lens, case.block_tables,
                        case.softmax_scale)
    assert (out[0] == 0).all() and np.isfinite(out[1]).all()
    del cache


@pytest.mark.parametrize("P", [16, 64, 512])
@pytest.mark.parametrize("window", [0, 100])
def test_split_partitions_merge_to_the_two_pass_result(P, window):
    case = workloads.make_case("split", 42, [1, 17, 511, 512, 513, 1300], [1] * 6, 8, 2, 128,
                               window=window)
    cache = build_cache(case)
    q = to_numpy(case.q())
    ref = oracle.decode(cache, q, "bf16", case.seq_lens, case.block_tables, case.softmax_scale, window)
    got = oracle.decode_split(cache, q, "bf16", case.seq_lens, case.block_tables,
                              case.softmax_scale, P, window)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_int8_kv_output_keeps_cosine_above_098():
    """MicroGen (Key Features) states >0.98 cosine similarity for its dynamic
    INT8 KV cache; here it is checked on the attention output, per vector."""
    case = workloads.qwen_decode(batch=8, seed=4, kv_dtype="i8", outliers=0.01)
    out_q = expected_outputs(case)                      # INT8 pool, dequantised as q * s
    out_f = expected_outputs(case, kv_dtype="bf16")     # the same K/V unquantised
    a = out_q.reshape(-1, case.head_dim)
    b = out_f.reshape(-1, case.head_dim)
    cos = (a * b).sum(1) / np.linalg.norm(a, axis=1) / np.linalg.norm(b, axis=1)
    assert cos.min() > 0.98, cos.min()
    assert not np.array_equal(out_q, out_f)
