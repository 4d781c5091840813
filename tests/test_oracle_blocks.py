"""Pins of the oracle's slot mapping and block copy.

Slot mapping ("MicroGen", Key Features: logical-to-physical block mapping;
"PyTorch LLM Serving Engine", Loading: each new K/V vector goes to a physical
cache slot): row i of a chunk of C rows of a sequence of L tokens sits at
position L - C + i.  Pinned by a round trip -- tokens written to the slots it
returns must be exactly what the (separately pinned) attention reads at those
positions, so the oracle's output equals dense causal attention on the
generated K/V -- by the closed form of an identity table, and by invariants
(distinct slots, each inside its own sequence's blocks, -1 where the table
holds no block).

Block copy (sharing a block between sequences before one writes into it):
pinned by numpy's own fancy-index copy of the pools, a swap (all sources are
read before any destination is written), and by attention invariance: a
sequence whose blocks are copied elsewhere and whose table is rewritten gives
bit-identical output.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle.cases import build_cache, expected_outputs, to_numpy


def _chunked(seq_lens, new_lens, window=0, seed=61, hq=8, hkv=2, d=64, dtype="bf16"):
    return workloads.make_case("blocks", seed, seq_lens, new_lens, hq, hkv, d, in_dtype=dtype,
                               window=window, kind="prefill")


def test_slot_mapping_round_trip_equals_dense_causal_attention():
    case = _chunked([37, 80, 16, 129], [5, 80, 1, 64])
    slots = oracle.slot_mapping(case.num_blocks, case.block_size, case.cu_q_lens, case.seq_lens,
                                case.block_tables)
    cache = build_cache(case, include_new=False)          # context tokens only
    cu = case.cu_q_lens
    for s in range(case.num_seqs):
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        k = to_numpy(case.kv("k", s, L - C, L))
        v = to_numpy(case.kv("v", s, L - C, L))
        cache.write(k, v, case.in_dtype, slots[cu[s]:cu[s + 1]])
    got = expected_outputs(case, cache=cache)
    for s in range(case.num_seqs):
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        q = case.q_seq(s).double().permute(1, 0, 2).unsqueeze(0)
        k = case.kv("k", s, 0, L).double().permute(1, 0, 2).unsqueeze(0)
        v = case.kv("v", s, 0, L).double().permute(1, 0, 2).unsqueeze(0)
        # rows at positions L-C .. L-1: a bottom-right aligned causal mask
        mask = torch.arange(L)[None, :] <= torch.arange(L - C, L)[:, None]
        ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(case.softmax_scale),
                                             enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref, rtol=0, atol=1e-12)


def test_slot_mapping_identity_table_is_base_plus_position():
    bs, nb, maxb = 16, 64, 8
    lens = np.array([1, 16, 17, 100], np.int32)
    new = np.array([1, 16, 3, 7], np.int32)
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    base = np.array([0, 7, 15, 23], np.int32)              # first block of each sequence
    tables = base[:, None] + np.arange(maxb, dtype=np.int32)[None, :]
    slots = oracle.slot_mapping(nb, bs, cu, lens, tables)
    for s in range(4):
        p = np.arange(lens[s] - new[s], lens[s])
        assert np.array_equal(slots[cu[s]:cu[s + 1]], base[s] * bs + p)


def test_slot_mapping_invariants_on_a_shuffled_pool():
    lens = workloads.lognormal_lengths(7, 40, 300, 1, 2000)
    new = np.minimum(lens, workloads.uniform_ints(8, 40, 1, 300)).astype(np.int32)
    case = _chunked(lens, new)
    slots = oracle.slot_mapping(case.num_blocks, case.block_size, case.cu_q_lens, case.seq_lens,
                                case.block_tables)
    assert slots.size == int(new.sum()) and (slots >= 0).all()
    assert np.unique(slots).size == slots.size                        # each slot written once
    assert np.array_equal(slots, case.new_slots())                    # the generator's own mapping
    cu = case.cu_q_lens
    for s in range(case.num_seqs):
        nblk = -(-int(lens[s]) // 16)
        own = set(case.block_tables[s, :nblk].tolist())
        assert set((slots[cu[s]:cu[s + 1]] // 16).tolist()) <= own


def test_slot_mapping_marks_missing_blocks():
    tables = np.array([[3, -1, 9], [50, 2, 2]], np.int32)            # -1, and 50 >= num_blocks
    lens = np.array([40, 20], np.int32)
    cu = np.array([0, 40, 42], np.int32)
    slots = oracle.slot_mapping(10, 16, cu, lens, tables)
    assert np.array_equal(slots[:16], 3 * 16 + np.arange(16))
    assert (slots[16:32] == -1).all()
    assert np.array_equal(slots[32:40], 9 * 16 + np.arange(8))
    assert np.array_equal(slots[40:], [2 * 16 + 2, 2 * 16 + 3])
    # a chunk longer than the sequence: rows before position 0 have no slot
    slots = oracle.slot_mapping(10, 16, np.array([0, 5], np.int32), np.array([3], np.int32), tables[:1])
    assert np.array_equal(slots, [-1, -1, 48, 49, 50])


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_copy_blocks_equals_numpy_copy(kv_dtype):
    case = workloads.make_case("copy", 62, [40, 70], [1, 1], 4, 2, 64, in_dtype="f32" if kv_dtype == "f32" else "bf16",
                               kv_dtype=kv_dtype, num_blocks=16)
    cache = build_cache(case)
    before = [x.copy() for x in (cache.k, cache.v, cache.k_scale, cache.v_scale) if x is not None]
    src = np.array([case.block_tables[0, 0], case.block_tables[1, 2], 5, 99], np.int32)
    dst = np.array([case.block_tables[1, 2], case.block_tables[0, 0], 11, 3], np.int32)  # a swap, a copy, a bad id
    oracle.copy_blocks(cache, src, dst)
    after = [x for x in (cache.k, cache.v, cache.k_scale, cache.v_scale) if x is not None]
    for b, a in zip(before, after):
        ref = b.copy()
        ref[dst[:3]] = b[src[:3]]
        assert np.array_equal(a.view(np.uint8), ref.view(np.uint8))


def test_copied_blocks_attend_identically():
    case = workloads.make_case("copy", 63, [50, 33, 90], [1, 1, 1], 8, 2, 64, num_blocks=40)
    cache = build_cache(case)
    ref = expected_outputs(case, cache=cache)
    used = set(case.block_tables[:, :].ravel().tolist())
    free = [b for b in range(case.num_blocks) if b not in used]
    nblk = -(-int(case.seq_lens[2]) // 16)
    src = case.block_tables[2, :nblk].copy()
    dst = np.array(free[:nblk], np.int32)
    oracle.copy_blocks(cache, src, dst)
    cache.k[src] = 0x7FC0                              # the originals are gone
    cache.v[src] = 0x7FC0
    case.block_tables[2, :nblk] = dst
    got = expected_outputs(case, cache=cache)
    assert np.array_equal(got, ref)


def _sdpa_rows_with_absent_blocks(case, s, absent_cols):
    """Dense fp64 attention (torch SDPA) of sequence s's query rows over its
    generated K/V, causal and windowed, with the keys of the logical blocks in
    absent_cols removed from every row; rows with no key left are zero."""
    L, C = int(case.seq_lens[s]), int(case.new_lens[s])
    W = case.window
    q = case.q_seq(s).double().permute(1, 0, 2).unsqueeze(0)
    k = case.kv("k", s, 0, L).double().permute(1, 0, 2).unsqueeze(0)
    v = case.kv("v", s, 0, L).double().permute(1, 0, 2).unsqueeze(0)
    pos = torch.arange(L - C, L)[:, None]
    key = torch.arange(L)[None, :]
    mask = key <= pos
    if W > 0:
        mask &= key > pos - W
    present = torch.ones(L, dtype=torch.bool)
    for c in absent_cols:
        present[c * 16:(c + 1) * 16] = False
    mask &= present[None, :]
    empty = ~mask.any(1)
    mask[empty, 0] = True                       # SDPA needs a key per row; those rows are zeroed below
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(case.softmax_scale),
                                         enable_gqa=True)[0].permute(1, 0, 2).numpy()
    ref[empty.numpy()] = 0.0
    return ref


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_missing_blocks_before_the_window_change_nothing(kind):
    """Window eviction releases the blocks wholly before every query's window and
    marks their table entries -1 ("MicroGen", Key Features: window-length
    eviction); the oracle must give the same output without reading them.  A
    released block that a query could still see holds no keys for it: the
    output is attention over the keys that remain (torch SDPA with that
    block's keys masked out)."""
    W = 40
    lens, new = [300, 97, 64], ([1, 1, 1] if kind == "decode" else [20, 30, 64])
    case = workloads.make_case("evict", 64, lens, new, 8, 2, 64, window=W, kind=kind)
    cache = build_cache(case)
    ref = expected_outputs(case, cache=cache)
    evicted = case.block_tables.copy()
    for s in range(case.num_seqs):
        first_query = int(case.seq_lens[s]) - int(case.new_lens[s])
        dead = max(0, first_query - W + 1) // 16
        evicted[s, :dead] = -1
    assert (evicted == -1).any()
    case.block_tables = evicted
    assert np.array_equal(expected_outputs(case, cache=cache), ref)
    # one more block, still inside a window: the rows that saw it now attend
    # over the remaining keys only
    s = 0
    first_query = int(case.seq_lens[s]) - int(case.new_lens[s])
    col = max(0, first_query - W + 1) // 16
    evicted[s, col] = -1
    got = expected_outputs(case, cache=cache)
    cu = case.cu_q_lens
    sdpa = _sdpa_rows_with_absent_blocks(case, s, [col])
    np.testing.assert_allclose(got[cu[s]:cu[s + 1]], sdpa, rtol=0, atol=1e-12)
    assert not np.allclose(got[cu[s]:cu[s + 1]], ref[cu[s]:cu[s + 1]])


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_entries_without_a_block_hold_no_keys(kind):
    """A table entry that is not a block of the pool (-1, or an id past the pool)
    inside the visible range holds no keys: the oracle equals dense attention
    over the keys that remain, and a row left with no key is zero (like an
    empty context).  Covers single and split-K decode."""
    lens = [100, 40, 33, 16]
    new = [1] * 4 if kind == "decode" else [30, 40, 10, 16]
    case = workloads.make_case("absent", 65, lens, new, 8, 2, 64, kind=kind)
    cache = build_cache(case)
    holes = {0: [1, 3], 1: [0], 2: [2], 3: [0]}        # sequence 3 loses its only block
    t = case.block_tables.copy()
    for s, cols in holes.items():
        for c in cols:
            t[s, c] = -1 if c % 2 == 0 else case.num_blocks + 5
    case.block_tables = t
    got = expected_outputs(case, cache=cache)
    cu = case.cu_q_lens
    for s, cols in holes.items():
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], _sdpa_rows_with_absent_blocks(case, s, cols),
                                   rtol=0, atol=1e-12)
    assert (got[cu[3]:cu[4]] == 0).all()
    if kind == "decode":
        q = to_numpy(case.q())
        for part in (16, 32):
            split = oracle.decode_split(cache, q, case.in_dtype, case.seq_lens, t, case.softmax_scale, part)
            np.testing.assert_allclose(split, got, rtol=0, atol=1e-12)


def test_logical_tables_of_offset_rows():
    rows = np.array([[5, 6, 7], [9, -1, 3]], np.int32)
    got = oracle.logical_tables(rows, np.array([2, 0], np.int32))
    assert np.array_equal(got, [[-1, -1, 5, 6, 7], [9, -1, 3, -1, -1]])
    assert np.array_equal(oracle.logical_tables(rows), rows)


def _compact(case, W):
    """Offset rows: drop each sequence's blocks wholly before its first query's
    window; the narrower rows are padded with an id that is never read."""
    offs, rows = [], []
    for s in range(case.num_seqs):
        first_query = int(case.seq_lens[s]) - int(case.new_lens[s])
        offs.append(max(0, first_query - W + 1) // 16)
        nblk = -(-int(case.seq_lens[s]) // 16)
        rows.append(case.block_tables[s, offs[-1]:nblk])
    width = max(len(r) for r in rows)
    out = np.full((case.num_seqs, width), 7777, np.int32)
    for s, r in enumerate(rows):
        out[s, :len(r)] = r
    return out, np.array(offs, np.int32)


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_offset_tables_give_the_same_attention_and_slots(kind):
    """A row whose column c holds logical block c + offset ("MicroGen", Key
    Features: window eviction; the table keeps only the window's blocks)."""
    W = 48
    lens, new = [700, 97, 64, 300], ([1, 1, 1, 1] if kind == "decode" else [20, 30, 64, 5])
    case = workloads.make_case("offset", 65, lens, new, 8, 2, 64, window=W, kind=kind)
    cache = build_cache(case)
    ref = expected_outputs(case, cache=cache)
    rows, offs = _compact(case, W)
    assert offs.max() > 0 and rows.shape[1] < case.block_tables.shape[1]
    q = to_numpy(case.q())
    if kind == "decode":
        got = oracle.decode(cache, q, case.in_dtype, case.seq_lens, rows, case.softmax_scale, W, table_offsets=offs)
    else:
        got = oracle.attention(cache, q, case.in_dtype, case.cu_q_lens, case.seq_lens, rows, case.softmax_scale, W,
                               table_offsets=offs)
    assert np.array_equal(got, ref)
    a = oracle.slot_mapping(case.num_blocks, 16, case.cu_q_lens, case.seq_lens, case.block_tables)
    b = oracle.slot_mapping(case.num_blocks, 16, case.cu_q_lens, case.seq_lens, rows, table_offsets=offs)
    assert np.array_equal(a, b)
