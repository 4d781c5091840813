"""The order in which the GPU kernels visit keys, replayed on the host from a
case's inputs, to show that a test input really drives the online softmax
through its rescale branch (a later group of keys outscoring, by more than the
lazy threshold of 2^8, everything the same running state has seen before).

Scores are computed in fp64 from the inputs as handed to the cache write
(rounded to the input dtype; an INT8 pool's quantisation moves them by far
less than the margin used here).  A sufficient condition is checked, not the
kernels' exact decision: a running maximum never exceeds the largest score its
state has seen, so a key group whose maximum passes every earlier group's by
more than 8 + margin (log2 units) is certain to trigger the rescale, whatever
the kernel's rounding.

Decode (`paged_attention_decode`): a work item is (sequence, partition, KV
head); the keys of the partition are taken in batches that end at multiples
of 4096 positions, each batch's 16-token blocks dealt to the 4 waves
round-robin from the batch's first block; each wave keeps its own state over
all its blocks of the item.  Prefill (`paged_attention_prefill_chunk`): a
workgroup owns 256 rows (chunk token, query head of the group) of one
(sequence, KV head); all its rows meet the same 64-key tiles, from the first
64-key boundary at or before the earliest row's first visible key.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
THRESHOLD = 8.0
BATCH_KEYS = 4096
WAVES = 4
ROWS_PER_WG = 256
TILE_KEYS = 64


def _scores(case, s, g, rows_q, L):
    """log2-unit scores [rows][L] of query rows (fp64) against the keys of KV head g."""
    k = case.kv("k", s, 0, L).double()[:, g].numpy()          # [L][D]
    return (rows_q @ k.T) * float(case.softmax_scale) * LOG2E


def _first_visible(p, window):
    return max(0, p - window + 1) if window > 0 else 0


def _jump_after_first(groups, margin):
    """groups: list of 1-D arrays of scores, in visiting order (empty = no key).
    True if some group's maximum passes the maximum of every earlier group by
    more than THRESHOLD + margin, with an earlier group holding a key."""
    best = -np.inf
    for grp in groups:
        if grp.size == 0:
            continue
        m = grp.max()
        if best > -np.inf and m > best + THRESHOLD + margin:
            return True
        best = max(best, m)
    return False


def decode_wave_groups(case, s, L, partition_size):
    """For sequence s (context L), the key positions each wave visits, per item
    (partition): a list over partitions of a list over waves of lists of
    per-block position arrays."""
    lo = _first_visible(L - 1, case.window)
    P = partition_size
    if P > 0:
        parts = [(max(lo, k * P), min(L, (k + 1) * P)) for k in range(lo // P, (L - 1) // P + 1)]
    else:
        parts = [(lo, L)]
    out = []
    for t0, t1 in parts:
        waves = [[] for _ in range(WAVES)]
        c0 = t0
        while c0 < t1:
            c1 = min(t1, (c0 // BATCH_KEYS + 1) * BATCH_KEYS)
            b0 = c0 // 16
            for b in range(b0, (c1 - 1) // 16 + 1):
                keys = np.arange(max(c0, b * 16), min(c1, b * 16 + 16))
                waves[(b - b0) % WAVES].append(keys)
            c0 = c1
        out.append(waves)
    return out


def decode_rows_reaching_rescale(case, partition_size, margin=1.0):
    """bool [num_seqs][num_q_heads]: the row's partition kernel certainly takes
    the rescale branch in some wave of some item."""
    q = case.q().double().numpy()
    G = case.group
    res = np.zeros((case.num_seqs, case.num_q_heads), bool)
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        if L == 0:
            continue
        items = decode_wave_groups(case, s, L, partition_size)
        for g in range(case.num_kv_heads):
            sc = _scores(case, s, g, q[s, g * G:(g + 1) * G], L)
            for j in range(G):
                for waves in items:
                    if any(_jump_after_first([sc[j, blk] for blk in w], margin) for w in waves):
                        res[s, g * G + j] = True
                        break
    return res


def decode_rows_merging_spread_partitions(case, partition_size, margin=1.0):
    """bool [num_seqs][num_q_heads]: the merge kernel combines partitions whose
    maxima lie more than 8 + margin (log2 units) apart."""
    q = case.q().double().numpy()
    G = case.group
    res = np.zeros((case.num_seqs, case.num_q_heads), bool)
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        if L == 0:
            continue
        lo = _first_visible(L - 1, case.window)
        P = partition_size
        for g in range(case.num_kv_heads):
            sc = _scores(case, s, g, q[s, g * G:(g + 1) * G], L)
            for j in range(G):
                m = [sc[j, max(lo, k * P):min(L, (k + 1) * P)].max() for k in range(lo // P, (L - 1) // P + 1)]
                res[s, g * G + j] = len(m) > 1 and max(m) - min(m) > THRESHOLD + margin
    return res


def prefill_rows_reaching_rescale(case, margin=1.0):
    """bool [total_rows][num_q_heads]: the row takes the rescale branch on some tile."""
    q = case.q().double().numpy()
    G = case.group
    res = np.zeros((case.total_q, case.num_q_heads), bool)
    cu = case.cu_q_lens
    for s in range(case.num_seqs):
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        if C == 0:
            continue
        base = L - C
        for g in range(case.num_kv_heads):
            rows_q = q[cu[s]:cu[s + 1], g * G:(g + 1) * G].reshape(C * G, -1)     # row = tok * G + jh
            sc = _scores(case, s, g, rows_q, L)
            for r0 in range(0, C * G, ROWS_PER_WG):
                p_min = base + r0 // G
                p_max = base + (min(C * G, r0 + ROWS_PER_WG) - 1) // G
                kt0 = (_first_visible(p_min, case.window) // TILE_KEYS) * TILE_KEYS
                for r in range(r0, min(C * G, r0 + ROWS_PER_WG)):
                    p = base + r // G
                    lo = _first_visible(p, case.window)
                    groups = []
                    for kt in range(kt0, p_max + 1, TILE_KEYS):
                        a, b = max(kt, lo), min(kt + TILE_KEYS - 1, p)
                        groups.append(sc[r, a:b + 1] if b >= a else np.zeros(0))
                    res[cu[s] + r // G, g * G + r % G] = _jump_after_first(groups, margin)
    return res
