"""GPU paged_attention_prefill_chunk against the fp64 oracle.

Chunks of new tokens are written through kv_cache_write into a NaN-poisoned,
block-shuffled pool, then attended with causal and sliding-window masks on
bf16 MFMA; sizes span several 256-row and 64-key tiles with ragged tails."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.cases import build_cache, expected_outputs, to_numpy
from pkv_testlib import alloc_pools, assert_close, bf16_ulp, device, run_prefill, write_tokens

pytestmark = pytest.mark.gpu


def _case(seq_lens, new_lens, hq=8, hkv=2, d=128, window=0, seed=81):
    return workloads.make_case("prefill", seed, seq_lens, new_lens, hq, hkv, d, window=window, kind="prefill")


def _gpu(case, **kw):
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "all")
    out = run_prefill(case, pools, dev, **kw)
    torch.cuda.synchronize()
    return out, pools


SHAPES = [  # seq_lens, new_lens
    ([40, 17, 300], [40, 17, 300]),           # whole sequences from position 0
    ([1, 2, 33, 64, 65], [1, 2, 30, 5, 65]),
    ([1000, 700, 129], [256, 100, 33]),
    ([2100, 64], [31, 64]),
]


@pytest.mark.parametrize("lens,new", SHAPES, ids=["from0", "small", "mid", "long"])
@pytest.mark.parametrize("window", [0, 1, 17, 100, 512])
def test_prefill_matches_oracle(lens, new, window):
    case = _case(lens, new, window=window)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", f"W={window}")


@pytest.mark.parametrize("window", [0, 4096])
def test_prefill_large_chunk_many_row_tiles(window):
    """A 1024-token chunk (4096 query rows with 4 q heads per KV head: 16 row
    tiles of one (sequence, KV head)) on a 4200-token sequence, beside a whole
    700-token sequence; with the 4096-token window the chunk's early rows see
    keys from position 0 and its late rows start past it."""
    case = _case([4200, 700], [1024, 700], window=window, seed=80)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", f"W={window}")


GEOMS = [(4, 4, 128), (8, 2, 64), (12, 2, 128), (6, 1, 64), (32, 8, 128), (16, 2, 128), (5, 5, 64)]


@pytest.mark.parametrize("hq,hkv,d", GEOMS, ids=[f"{g[0]}q{g[1]}kv-D{g[2]}" for g in GEOMS])
def test_prefill_group_sizes_and_head_dims(hq, hkv, d):
    case = _case([300, 77, 1500], [130, 77, 40], hq=hq, hkv=hkv, d=d, window=200)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16")


def test_prefill_bf16_output():
    case = _case([400, 90], [200, 90], window=128)
    out, _ = _gpu(case, out_dtype=torch.bfloat16)
    ref = expected_outputs(case)
    got = out.float().cpu().double().numpy()
    assert (np.abs(got - ref) <= bf16_ulp(ref) + 2e-3).all()


def test_prefill_block_permutation_and_reruns_are_bit_identical():
    case = _case([600, 250], [256, 250], window=300)
    a, pools = _gpu(case)
    b = run_prefill(case, pools, device())
    c, _ = _gpu(case.subset(range(case.num_seqs)))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, c)


def test_prefill_single_row_chunks_match_decode_semantics():
    case = _case([5, 300, 1029], [1, 1, 1], hq=8, hkv=2, window=0)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16")


def _every_wave_rows(case):
    """Chunk tokens that put a checked row in every wave of every row tile of
    every (sequence, KV head) at the benchmark's launch shape (256 rows of
    (token, query head) per workgroup, 32 per wave, so 8 tokens per wave with
    G = 4): token 8w + (w % 8) of wave w, at a different lane each time."""
    rows_per_wave = 32 // case.group
    return [w * rows_per_wave + (w % rows_per_wave) for w in range(-(-int(case.new_lens.max()) // rows_per_wave))]


def _check_rows_by_prefix_decode(case, out, kind):
    """Each chosen chunk row against the oracle's decode over its prefix (pinned
    equal to chunk rows), all rows of a sequence in one oracle call."""
    picks = list(range(case.num_seqs))
    toks = _every_wave_rows(case)
    cache = build_cache(case, device=device())
    q = to_numpy(case.q(device()))
    cu = case.cu_q_lens
    worst = 0.0
    for s in picks:
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        ii = [i for i in toks if i < C]
        rows = np.array([cu[s] + i for i in ii])
        lens = np.array([L - C + i + 1 for i in ii], np.int32)
        # each row's table starts at the block of its first visible key (offset
        # rows), so the oracle gathers its window rather than the whole context
        offs = np.array([max(0, int(n) - case.window) // 16 if case.window > 0 else 0 for n in lens], np.int32)
        tables = np.stack([np.concatenate([case.block_tables[s, o:], np.full(o, -1, np.int32)]) for o in offs])
        ref = oracle.decode(cache, q[rows], "bf16", lens, tables, case.softmax_scale, case.window,
                            table_offsets=offs)
        worst = max(worst, assert_close(out[torch.from_numpy(rows).to(out.device)], ref, "bf16",
                                        f"{kind} seq {s}"))
    return worst


def test_prefill_window_4096_full_size_every_wave():
    """16 sequences x 256 new tokens on 1024..16384-token contexts, window 4096,
    32 q / 8 kv heads -- the benchmark's launch configuration.  One row in every
    (sequence, KV head, row tile, wave) is checked against the oracle (all 32
    query heads of 32 tokens per sequence)."""
    case = workloads.prefill_window()
    out, _ = _gpu(case)
    assert torch.isfinite(out).all()
    err = _check_rows_by_prefix_decode(case, out, "bf16")
    print(f"window-4096 prefill: {len(_every_wave_rows(case))} tokens per sequence checked, max abs error {err:.3e}")


def test_prefill_zero_scale_and_empty_chunks():
    case = workloads.make_case("z", 82, [50, 20, 70], [0, 20, 5], 8, 2, 128, softmax_scale=0.0,
                               window=10, kind="prefill")
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16")


# ---------------------------------------------------------------- INT8 pools
def _i8(seq_lens, new_lens, hq=8, hkv=2, d=128, window=0, seed=91, **kw):
    return workloads.make_case("prefill-i8", seed, seq_lens, new_lens, hq, hkv, d, kv_dtype="i8",
                               outliers=0.01, window=window, kind="prefill", **kw)


@pytest.mark.parametrize("lens,new", SHAPES, ids=["from0", "small", "mid", "long"])
@pytest.mark.parametrize("window", [0, 17, 512])
def test_int8_prefill_matches_dequantised_oracle(lens, new, window):
    """K/V written through the quantising cache write (1% x8 outliers); the
    oracle attends over the same dequantised cache ("MicroGen", Key Features:
    dynamic INT8 KV)."""
    case = _i8(lens, new, window=window)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", f"int8 W={window}")


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (12, 2, 128), (5, 5, 64), (32, 8, 128)])
def test_int8_prefill_geometries_and_cosine(hq, hkv, d):
    case = _i8([300, 77, 1100], [130, 77, 40], hq=hq, hkv=hkv, d=d, window=200)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", "int8")
    ref_f = expected_outputs(case, kv_dtype="bf16")        # the same K/V unquantised
    a = out.double().cpu().numpy().reshape(-1, d)
    b = ref_f.reshape(-1, d)
    cos = (a * b).sum(1) / np.linalg.norm(a, axis=1) / np.linalg.norm(b, axis=1)
    assert cos.min() > 0.98, cos.min()


def test_int8_prefill_zero_scale_empty_chunks_and_bf16_output():
    case = _i8([50, 20, 70], [0, 20, 5], window=10, softmax_scale=0.0)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", "int8 zero scale")
    case = _i8([400, 90], [200, 90], window=128)
    out, _ = _gpu(case, out_dtype=torch.bfloat16)
    ref = expected_outputs(case)
    got = out.float().cpu().double().numpy()
    assert (np.abs(got - ref) <= bf16_ulp(ref) + 2e-3).all()


def test_int8_prefill_window_4096_full_size_every_wave():
    """The window-4096 launch (16 x 256 rows on 1024..16384-token contexts,
    32 q / 8 kv heads) over an INT8 pool; one row in every (sequence, KV head,
    row tile, wave) against the oracle's decode over the matching prefix of the
    dequantised cache."""
    import dataclasses
    case = dataclasses.replace(workloads.prefill_window(), kv_dtype="i8", outliers=0.01)
    out, _ = _gpu(case)
    assert torch.isfinite(out).all()
    _check_rows_by_prefix_decode(case, out, "int8")


# ---------------------------------------------------------------- mixed batches
@pytest.mark.parametrize("window", [0, 300])
def test_mixed_decode_and_prefill_batch_in_one_launch(window):
    """Decode rows (chunks of one token) and prefill chunks in the same launch
    ("PyTorch LLM Serving Engine", What is implemented: prefill chunks share the
    step with decode work)."""
    lens = [900, 40, 1, 2000, 17, 333, 64, 1500, 250, 5]
    new = [128, 1, 1, 1, 17, 1, 64, 200, 1, 1]
    case = _case(lens, new, hq=12, hkv=2, window=window)
    out, _ = _gpu(case)
    assert_close(out, expected_outputs(case), "bf16", f"mixed W={window}")


def test_mixed_step_full_size_sampled_rows():
    """The mixed serving step at full size (16 chunks of 256 + 240 decode rows,
    32 q / 8 kv heads, window 4096): sampled decode rows and chunk rows against
    the oracle's decode over the matching prefix (pinned equal to chunk rows)."""
    case = workloads.mixed_step()
    out, _ = _gpu(case)
    assert torch.isfinite(out).all()
    picks = [0, 7, 15] + list(range(16, case.num_seqs, 9))
    sub = case.subset(picks)
    cache = build_cache(sub, device=device())
    q = to_numpy(sub.q(device()))
    cu = case.cu_q_lens
    for si, s in enumerate(picks):
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        for i in sorted({0, C - 1, C // 2}):
            row = int(sub.cu_q_lens[si]) + i
            ref = oracle.decode(cache, q[row:row + 1], "bf16", np.array([L - C + i + 1], np.int32),
                                sub.block_tables[si:si + 1], sub.softmax_scale, sub.window)
            assert_close(out[cu[s] + i:cu[s] + i + 1], ref, "bf16", f"seq {s} row {i}")
