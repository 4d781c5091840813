"""GPU paged_attention_decode against the fp64 oracle.

Every case writes its context through kv_cache_write into a NaN-poisoned,
block-shuffled pool, then decodes; the oracle does the same on the host.
Sizes span several 512-token partitions and ragged tails; the
Llama-3-8B-shaped batch runs at full size with sampled sequences checked."""
import numpy as np
import pytest
import torch

import workloads
from oracle.cases import build_cache, expected_outputs
from pkv_testlib import alloc_pools, assert_close, bf16_ulp, device, run_decode, write_tokens

pytestmark = pytest.mark.gpu


def _gpu(case, **kw):
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "context")
    write_tokens(case, pools, dev, "new")          # the step's own token, written first
    out = run_decode(case, pools, dev, **kw)
    torch.cuda.synchronize()
    return out, pools


def test_tiny_fp32_decode():
    case = workloads.tiny_fp32_decode()
    for part in (0, 16, 512):
        out, _ = _gpu(case, partition_size=part)
        assert_close(out, expected_outputs(case), "f32", f"partition {part}")


def test_qwen_shaped_bf16_decode():
    case = workloads.qwen_decode()
    ref = expected_outputs(case)
    for part in (512, 0, 64):
        out, _ = _gpu(case, partition_size=part)
        assert_close(out, ref, "bf16", f"partition {part}")


def test_int8_decode_matches_dequantised_oracle_and_keeps_cosine():
    case = workloads.int8_decode()
    out, _ = _gpu(case)
    ref_q = expected_outputs(case)                      # attention on the dequantised INT8 cache
    assert_close(out, ref_q, "bf16", "int8 vs dequantised oracle")
    ref_f = expected_outputs(case, kv_dtype="bf16")     # same K/V unquantised
    a = out.double().cpu().numpy().reshape(-1, case.head_dim)
    b = ref_f.reshape(-1, case.head_dim)
    cos = (a * b).sum(1) / np.linalg.norm(a, axis=1) / np.linalg.norm(b, axis=1)
    assert cos.min() > 0.98, cos.min()


@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
def test_int8_pool_with_either_query_dtype(q_dtype):
    case = workloads.make_case("i8q", 71, [1, 17, 600], [1, 1, 1], 8, 2, 64, in_dtype=q_dtype,
                               kv_dtype="i8", outliers=0.01)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", q_dtype)


GEOMS = [  # Hq, Hkv, D, dtype
    (8, 8, 128, "bf16"), (8, 4, 128, "bf16"), (9, 3, 128, "bf16"), (10, 2, 128, "bf16"),
    (14, 2, 64, "bf16"), (16, 2, 128, "bf16"), (12, 1, 128, "bf16"), (24, 2, 64, "bf16"),
    (71, 1, 64, "bf16"), (4, 4, 128, "f32"), (6, 1, 128, "f32"), (16, 8, 64, "f32"),
]


@pytest.mark.parametrize("hq,hkv,d,dt", GEOMS, ids=[f"{g[0]}q{g[1]}kv-D{g[2]}-{g[3]}" for g in GEOMS])
def test_group_sizes_and_head_dims(hq, hkv, d, dt):
    lens = [1, 2, 16, 17, 511, 512, 513, 1030]
    case = workloads.make_case("geom", 72, lens, [1] * len(lens), hq, hkv, d, in_dtype=dt)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), dt)


I8_GEOMS = [  # Hq, Hkv: query heads per KV head 1, 2, 3, 5, 8 at head_dim 128
    (4, 4), (8, 4), (9, 3), (10, 2), (16, 2),
]


@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hq,hkv", I8_GEOMS, ids=[f"{g[0]}q{g[1]}kv" for g in I8_GEOMS])
def test_int8_group_sizes_at_head_dim_128(hq, hkv, q_dtype):
    """INT8 pools at head_dim 128 for every group width the kernels handle in
    groups of four heads (fewer than four, more than four, two groups), with
    ragged lengths across 512-token partitions, single-pass and split."""
    lens = [1, 2, 16, 17, 511, 512, 513, 1030]
    case = workloads.make_case("i8geom", 74, lens, [1] * len(lens), hq, hkv, 128, in_dtype=q_dtype,
                               kv_dtype="i8", outliers=0.01)
    ref = expected_outputs(case)
    for part in (0, 512):
        out, _ = _gpu(case, partition_size=part)
        assert_close(out, ref, "bf16", f"{q_dtype} P={part}")


@pytest.mark.parametrize("window", [1, 7, 16, 500, 4096])
@pytest.mark.parametrize("part", [0, 16, 512])
def test_sliding_window(window, part):
    lens = [1, 5, 16, 40, 513, 1500, 2100]
    case = workloads.make_case("win", 73, lens, [1] * len(lens), 8, 2, 128, window=window)
    out, _ = _gpu(case, partition_size=part)
    assert_close(out, expected_outputs(case), "bf16", f"W={window} P={part}")


@pytest.mark.parametrize("dt,kv", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "i8")])
@pytest.mark.parametrize("window", [0, 5000])
def test_long_contexts_in_one_pass(dt, kv, window):
    """partition_size 0: one item walks the whole context, so its block ids come
    in several batches (4096 keys each); lengths straddle the batch edges and
    the window starts inside a batch."""
    lens = [4095, 4096, 4097, 9000, 12345]
    case = workloads.make_case("long", 78, lens, [1] * len(lens), 8, 2, 128, in_dtype=dt, kv_dtype=kv,
                               window=window)
    out, _ = _gpu(case, partition_size=0)
    assert_close(out, expected_outputs(case), dt, f"{kv} W={window}")


def test_empty_context_rows_are_zero():
    case = workloads.make_case("empty", 74, [0, 3, 0, 700], [1] * 4, 8, 2, 128)
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "all")
    for part in (0, 512):
        out = run_decode(case, pools, dev, partition_size=part)
        torch.cuda.synchronize()
        assert (out[0] == 0).all() and (out[2] == 0).all()
        ref = expected_outputs(case)
        assert_close(out, ref, "bf16")


def test_bf16_output_is_within_one_ulp_of_the_rounded_oracle():
    case = workloads.make_case("bf16out", 75, [33, 700, 1200], [1] * 3, 8, 2, 128)
    out, _ = _gpu(case, out_dtype=torch.bfloat16)
    ref = expected_outputs(case)
    got = out.float().cpu().double().numpy()
    assert (np.abs(got - ref) <= bf16_ulp(ref) + 2e-3).all()


def test_block_permutation_and_reruns_are_bit_identical():
    case = workloads.make_case("perm", 76, [100, 1000, 1600], [1] * 3, 16, 4, 128)
    a, pools = _gpu(case)
    b = run_decode(case, pools, device())
    compact, _ = _gpu(case.subset(range(case.num_seqs)))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, compact)


def test_more_sequences_than_one_launch_holds():
    lens = list(np.arange(2500) % 37 + 1)
    case = workloads.make_case("many", 77, lens, [1] * len(lens), 4, 2, 64)
    out, _ = _gpu(case, partition_size=16)
    assert_close(out, expected_outputs(case), "bf16")


def test_llama_shaped_full_size_every_sequence():
    """The full Llama-3-8B-shaped batch (256 sequences, ~840k tokens, 4 GB of
    pool) in the benchmark's launch configuration (512-token partitions), every
    output row checked against the oracle over the whole cache."""
    case = workloads.llama_decode()
    out, _ = _gpu(case)
    ref = expected_outputs(case, cache=build_cache(case, device=device()))
    err = assert_close(out, ref, "bf16", "all 256 sequences")
    print(f"llama-shaped decode: {case.num_seqs} sequences, max abs error {err:.3e}")


def test_longest_context_of_the_llama_shaped_range():
    """Contexts at the top of the Llama-shaped length range (32768 tokens) and
    one past it, beside one-block ones, with that workload's group of 4 q heads
    per KV head, head_dim 128 and 512-token partitions: the long rows have 64
    and 65 partitions, one more than the merge kernel's wave holds at once."""
    lens = [32768, 32769, 1, 511, 512, 513]
    case = workloads.make_case("longest", 79, lens, [1] * len(lens), 8, 2, 128)
    out, _ = _gpu(case, partition_size=512)
    assert_close(out, expected_outputs(case), "bf16", "part=512")
