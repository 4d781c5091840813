"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of pkv_oracle.c (on the CPU, in a
temporary directory), loads the mutant in place of the oracle and runs the
pins that should reject it.  A mutant that every pin accepts fails the test.
"""
import contextlib
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_attention as A
import test_oracle_blocks as BL
import test_oracle_int8 as Q
import test_oracle_numbers as N
import test_oracle_prefill as P

MUTANTS = [
    ("window off by one", "return p - window + 1;", "return p - window;",
     [A.test_window_of_one_returns_the_current_value_and_wide_window_is_no_window]),
    ("scale dropped", "scores[j] = scale * dot;", "scores[j] = dot;",
     [lambda: A.test_decode_equals_dense_sdpa(A.CASES[1], 0)]),
    ("no max subtraction", "Z += exp(scores[j] - m);", "Z += exp(scores[j]);",
     [A.test_huge_scores_stay_finite_and_pick_the_best_key]),
    ("interleaved GQA mapping", "for (int32_t h = g * G; h < (g + 1) * G; ++h) {\n                    for (int32_t d = 0; d < D; ++d)\n                        qv[d]",
     "for (int32_t h = g; h < num_q_heads; h += num_kv_heads) {\n                    for (int32_t d = 0; d < D; ++d)\n                        qv[d]",
     [lambda: A.test_decode_equals_dense_sdpa(A.CASES[1], 0)]),
    ("block table ignored", "int64_t blk = table_row[j / block_size];", "int64_t blk = j / block_size;",
     [lambda: A.test_decode_equals_dense_sdpa(A.CASES[0], 0)]),
    ("V replaced by K", "out[d] += w * V[", "out[d] += w * K[",
     [lambda: A.test_decode_equals_dense_sdpa(A.CASES[0], 0)]),
    ("KV head offset dropped in the write", "int64_t src = (int64_t)t * token_stride + (int64_t)h * head_dim;",
     "int64_t src = (int64_t)t * token_stride;",
     [lambda: A.test_decode_equals_dense_sdpa(A.CASES[0], 0)]),
    ("INT8 divisor 128", "a / 127.0f", "a / 128.0f",
     [lambda: Q.test_hand_worked_vectors(_golden("general"))]),
    ("INT8 ties away from zero", "double r = round_half_even(fabs((double)t));",
     "double r = floor(fabs((double)t) + 0.5);",
     [lambda: Q.test_hand_worked_vectors(_golden("exact ties"))]),
    ("fp16 ties away from zero", "double m = round_half_even((a * ldexp(1.0, -E) - 1.0) * 1024.0);",
     "double m = floor((a * ldexp(1.0, -E) - 1.0) * 1024.0 + 0.5);",
     [N.test_f32_to_f16_ties_go_to_even]),
    ("chunk rows at the wrong position", "const int32_t p = L - C + i;", "const int32_t p = i;",
     [lambda: P.test_each_chunk_row_equals_decode_over_its_prefix(0)]),
    ("no causal mask inside a chunk", "attend(qv, K, V, present, D, lo, p, scale, scores, o, w, L);",
     "attend(qv, K, V, present, D, lo, L - 1, scale, scores, o, w, L);",
     [lambda: P.test_whole_sequence_chunk_equals_causal_sdpa("bf16")]),
    ("merge weights dropped", "double wk = exp(mk - M);", "double wk = 1.0;",
     [lambda: A.test_split_partitions_merge_to_the_two_pass_result(64, 0)]),
    ("keys of missing blocks kept", "        if (!present[j]) continue;\n        double dot = 0.0;\n        for (int32_t d = 0; d < D; ++d) dot += qv[d] * K[(int64_t)j * D + d];\n        scores[j] = scale * dot;",
     "        double dot = 0.0;\n        for (int32_t d = 0; d < D; ++d) dot += qv[d] * K[(int64_t)j * D + d];\n        scores[j] = scale * dot;",
     [lambda: BL.test_entries_without_a_block_hold_no_keys("prefill")]),
    ("slot one position late", "int64_t p = (int64_t)seq_lens[s] - (r1 - r0) + (r - r0);",
     "int64_t p = (int64_t)seq_lens[s] - (r1 - r0) + (r - r0) + 1;",
     [BL.test_slot_mapping_round_trip_equals_dense_causal_attention,
      BL.test_slot_mapping_identity_table_is_base_plus_position]),
    ("slot offset in block dropped", "slot = (int32_t)((int64_t)blk * block_size + p % block_size);",
     "slot = (int32_t)((int64_t)blk * block_size);",
     [BL.test_slot_mapping_round_trip_equals_dense_causal_attention]),
    ("block copy reads its own writes", "for (int pass = 0; pass < 2; ++pass) {\n        for (int32_t n = 0; n < num_pairs; ++n) {",
     "for (int32_t n = 0; n < num_pairs; ++n) {\n        for (int pass = 0; pass < 2; ++pass) {",
     [lambda: BL.test_copy_blocks_equals_numpy_copy("bf16")]),
]


def _golden(name):
    import json
    return next(c for c in json.load(open(Q.GOLDEN))["cases"] if c["name"] == name)


@contextlib.contextmanager
def _mutant(old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "pkv_oracle.c")
        open(path, "w").write(src.replace(old, new))
        with open(os.path.join(d, "pkv_oracle.h"), "w") as h:
            h.write(open(os.path.join(oracle.HERE, "pkv_oracle.h")).read())
        so = os.path.join(d, "mutant.so")
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                        path, "-lm"], check=True)
        saved = oracle.lib()
        oracle._lib = oracle._declare(ctypes.CDLL(so))
        try:
            yield
        finally:
            oracle._lib = saved


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_the_mutant(name, old, new, pins):
    with _mutant(old, new):
        caught = 0
        for pin in pins:
            try:
                pin()
            except (AssertionError, ValueError):
                caught += 1
        assert caught == len(pins), f"mutant '{name}' passed a pin meant to reject it"
