"""GPU parity where the online softmax has to work for its result.

"PyTorch LLM Serving Engine", Loading: the attention keeps a running maximum
while it visits the blocks, so that the exponentials stay bounded however the
scores grow.  The kernels keep that maximum lazily: what has been accumulated
is rescaled only when a later key outscores the running maximum by more than
2^8.  With unit-variance inputs at the usual 1/sqrt(D) scale that almost never
happens after a wave's first tile, so these tests build inputs that force it:

  * scores that rise in steps along the context (workloads.rising_scores):
    every step of keys outscores everything before it by 2^12 (decode: in
    ascents of 512 positions, which keep the range of the scores, and so
    their fp32 rounding, bounded), and a host
    replay of each kernel's visiting order (kernel_order) asserts, from the
    inputs, that every output row meets the rescale (decode at 0 and 512-token
    partitions, prefill), or that its merge combines partitions whose maxima
    lie more than 2^8 apart (16-token partitions);
  * plain random inputs at softmax scales 1 and 4 (scores tens of log2 units
    apart, so the running maximum moves all the time);
  * a softmax scale of 1e4: the result must be finite and one-hot on the
    best key (the stability case);
  * V at the edges of the bf16 prefill path's fp16 range (|v| up to 60000,
    and below 2^-14), an INT8-pool decode query far outside binary16's range,
    and rows whose table entries hold no block.

Tolerances are those of pkv_testlib (bf16: abs 2e-3 and per-vector relative
1e-2; fp32: abs 1e-5), against the fp64 oracle on the same inputs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kernel_order as ko
import workloads
from oracle.cases import build_cache, expected_outputs
from pkv_testlib import alloc_pools, assert_close, device, run_decode, run_prefill, write_tokens

pytestmark = pytest.mark.gpu

DECODE_LENS = [700, 1300, 2100, 530, 4500]


def _decode_gpu(case, **kw):
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "all")
    out = run_decode(case, pools, dev, **kw)
    torch.cuda.synchronize()
    return out


def _prefill_gpu(case, **kw):
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "all")
    out = run_prefill(case, pools, dev, **kw)
    torch.cuda.synchronize()
    return out


DECODE_KINDS = {  # name: (Hq, Hkv, D, q/input dtype, pool dtype)
    "f32-G2": (4, 2, 64, "f32", "f32"),
    "bf16-G4": (8, 2, 128, "bf16", "bf16"),
    "bf16-G6": (12, 2, 128, "bf16", "bf16"),
    "i8-bf16q": (8, 2, 128, "bf16", "i8"),
    "i8-f32q": (8, 2, 128, "f32", "i8"),
}


@pytest.mark.parametrize("part", [0, 16, 512])
@pytest.mark.parametrize("kind", list(DECODE_KINDS))
def test_decode_rising_scores_take_the_rescale(kind, part):
    hq, hkv, d, dt, kv = DECODE_KINDS[kind]
    base = workloads.make_case("rise-dec", 101, DECODE_LENS, [1] * len(DECODE_LENS), hq, hkv, d, in_dtype=dt,
                               kv_dtype=kv)
    # one ascent of four 2^12 steps per 512 positions: every 512-token partition
    # climbs, and the scores stay within ~40 log2 units of each other
    case = workloads.rising_scores(base, stair=128, period=4)
    if part == 16:
        reach = ko.decode_rows_merging_spread_partitions(case, part)
    else:
        reach = ko.decode_rows_reaching_rescale(case, part)
    assert reach.all(), f"{(~reach).sum()} rows do not reach the rescale"
    out = _decode_gpu(case, partition_size=part)
    assert_close(out, expected_outputs(case), "f32" if kv == "f32" else "bf16", f"{kind} P={part}")


@pytest.mark.parametrize("window", [0, 500])
@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_prefill_rising_scores_take_the_rescale(kv, window):
    base = workloads.make_case("rise-pf", 102, [900, 1500, 2600], [256, 300, 64], 8, 2, 128, kv_dtype=kv,
                               window=window, kind="prefill")
    case = workloads.rising_scores(base)
    reach = ko.prefill_rows_reaching_rescale(case)
    assert reach.all(), f"{(~reach).sum()} rows do not reach the rescale"
    out = _prefill_gpu(case)
    assert_close(out, expected_outputs(case), "bf16", f"{kv} W={window}")


@pytest.mark.parametrize("scale", [1.0, 4.0])
@pytest.mark.parametrize("kind", ["bf16-G4", "i8-bf16q", "f32-G2"])
def test_decode_large_softmax_scales(kind, scale):
    """Unit-variance inputs at softmax scale 1 and 4: logits tens of log2 units
    apart, so running maxima move often; many rows meet the rescale."""
    hq, hkv, d, dt, kv = DECODE_KINDS[kind]
    case = workloads.make_case("bigscale", 103, DECODE_LENS, [1] * len(DECODE_LENS), hq, hkv, d, in_dtype=dt,
                               kv_dtype=kv, softmax_scale=scale)
    assert ko.decode_rows_reaching_rescale(case, 0).mean() > 0.5
    ref = expected_outputs(case)
    for part in (0, 512):
        out = _decode_gpu(case, partition_size=part)
        assert_close(out, ref, "f32" if kv == "f32" else "bf16", f"{kind} scale {scale} P={part}")


@pytest.mark.parametrize("scale", [1.0, 4.0])
@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_prefill_large_softmax_scales(kv, scale):
    case = workloads.make_case("bigscale-pf", 104, [900, 1500, 300], [256, 300, 300], 8, 2, 128, kv_dtype=kv,
                               softmax_scale=scale, window=700, kind="prefill")
    assert ko.prefill_rows_reaching_rescale(case).mean() > 0.4
    out = _prefill_gpu(case)
    assert_close(out, expected_outputs(case), "bf16", f"{kv} scale {scale}")


def _one_hot_rows(case, ref, rows_pos):
    """The oracle's rows equal V at the best visible key (up to rounding), and
    every row's best key beats the second by a wide margin, so the softmax at
    scale 1e4 leaves it the only weight."""
    q = case.q().double().numpy()
    G = case.group
    for s, row, p in rows_pos:
        lo = max(0, p - case.window + 1) if case.window > 0 else 0
        k = case.kv("k", s, 0, p + 1).double().numpy()
        v = case.kv("v", s, 0, p + 1).double().numpy()
        for h in range(case.num_q_heads):
            g = h // G
            sc = k[lo:, g] @ q[row, h]
            top = np.argsort(sc)[::-1]
            assert sc.size == 1 or sc[top[0]] - sc[top[1]] > 1e-3, "near tie: choose another seed"
            np.testing.assert_allclose(ref[row, h], v[lo + top[0], g], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["f32-G2", "bf16-G4", "i8-bf16q"])
def test_decode_huge_scale_is_finite_and_one_hot(kind):
    hq, hkv, d, dt, kv = DECODE_KINDS[kind]
    lens = [1, 2, 17, 700, 1300]
    case = workloads.make_case("onehot", 105, lens, [1] * len(lens), hq, hkv, d, in_dtype=dt, kv_dtype=kv,
                               softmax_scale=1e4)
    ref = expected_outputs(case)
    if kv != "i8":                       # INT8: the oracle's one-hot row is the dequantised V
        _one_hot_rows(case, ref, [(s, s, int(case.seq_lens[s]) - 1) for s in range(case.num_seqs)])
    for part in (0, 16, 512):
        out = _decode_gpu(case, partition_size=part)
        assert torch.isfinite(out).all()
        assert_close(out, ref, "f32" if kv == "f32" else "bf16", f"{kind} P={part}")


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_prefill_huge_scale_is_finite_and_one_hot(kv):
    case = workloads.make_case("onehot-pf", 106, [300, 1000], [300, 200], 8, 2, 128, kv_dtype=kv,
                               softmax_scale=1e4, window=600, kind="prefill")
    ref = expected_outputs(case)
    if kv == "bf16":
        cu = case.cu_q_lens
        rows = [(s, cu[s] + i, int(case.seq_lens[s]) - int(case.new_lens[s]) + i)
                for s in range(case.num_seqs) for i in (0, 1, 63, 64, int(case.new_lens[s]) - 1)]
        _one_hot_rows(case, ref, rows)
    out = _prefill_gpu(case)
    assert torch.isfinite(out).all()
    assert_close(out, ref, "bf16", f"{kv} scale 1e4")


# ---------------------------------------------------------------- V at the fp16 edges
def _scaled_v(case, factor, clip=None):
    """The case's inputs with V multiplied by `factor` (then clipped), as fp32."""
    ntok = int(case.tok_base[-1] + case.seq_lens[-1])
    hd = case.num_kv_heads * case.head_dim
    K = workloads.normal_f32(case.seed, workloads.TAG_K, 0, ntok * hd).view(ntok, case.num_kv_heads, -1)
    V = workloads.normal_f32(case.seed, workloads.TAG_V, 0, ntok * hd).view(ntok, case.num_kv_heads, -1) * factor
    if clip is not None:
        V = V.clamp(-clip, clip)
    Q = workloads.normal_f32(case.seed, workloads.TAG_Q, 0, case.total_q * case.num_q_heads * case.head_dim)
    return workloads.ExplicitCase.wrap(case, K, V, Q.view(case.total_q, case.num_q_heads, -1))


def test_prefill_and_decode_with_v_up_to_60000():
    """V scaled by 15000 and clipped to 60000 (inside fp16's range: the bf16
    prefill path converts V to fp16).  The output is linear in V and the
    softmax weights do not depend on it, so the comparison is made in units of
    the scale factor: the usual tolerances apply to out / 15000."""
    f = 15000.0
    pf = _scaled_v(workloads.make_case("bigv", 107, [300, 1000, 90], [300, 200, 90], 8, 2, 128, window=500,
                                       kind="prefill"), f, 60000.0)
    assert float(pf.V.abs().max()) >= 59000.0
    out = _prefill_gpu(pf)
    assert torch.isfinite(out).all()
    assert_close(out / f, expected_outputs(pf) / f, "bf16", "prefill |v| <= 60000")
    dec = _scaled_v(workloads.make_case("bigv-d", 108, [1, 300, 1000, 2100], [1] * 4, 8, 2, 128), f, 60000.0)
    ref = expected_outputs(dec)
    for part in (0, 512):
        out = _decode_gpu(dec, partition_size=part)
        assert_close(out / f, ref / f, "bf16", f"decode |v| <= 60000 P={part}")


def test_prefill_and_decode_with_v_below_fp16_normal_range():
    """V scaled by 2^-18, so every |v| < 2^-14: the bf16 prefill path keeps each
    value on fp16's subnormal grid, off by at most 2^-25, which bounds the
    output's absolute error by 2^-25 plus fp32 rounding (checked against
    2^-24); the relative bound is not promised there.  Decode has no such
    limit: it meets the usual tolerances in units of the scale factor."""
    f = 2.0 ** -18
    pf = _scaled_v(workloads.make_case("tinyv", 109, [300, 1000, 90], [300, 200, 90], 8, 2, 128, window=500,
                                       kind="prefill"), f)
    assert float(pf.V.abs().max()) < 2.0 ** -14
    out = _prefill_gpu(pf)
    ref = expected_outputs(pf)
    err = np.abs(out.double().cpu().numpy() - ref)
    assert np.isfinite(err).all() and err.max() <= 2.0 ** -24, err.max()
    dec = _scaled_v(workloads.make_case("tinyv-d", 110, [1, 300, 1000, 2100], [1] * 4, 8, 2, 128), f)
    ref = expected_outputs(dec)
    for part in (0, 512):
        out = _decode_gpu(dec, partition_size=part)
        assert_close(out / f, ref / f, "bf16", f"decode |v| < 2^-14 P={part}")


# ---------------------------------------------------------------- INT8 pools: query magnitude
@pytest.mark.parametrize("log2f", [18, 0, -30])
def test_int8_decode_query_far_outside_fp16_range(log2f):
    """INT8 pools with a bf16 query keep the query's full exponent range: Q
    multiplied by 2^log2f (2^18: |q| past binary16's largest finite value;
    2^-30: every |q| below its smallest normal) with the softmax scale divided
    by the same factor, so the weights stay those of the unscaled case; the
    usual tolerances apply."""
    f = 2.0 ** log2f
    base = workloads.make_case("i8qmag", 111, [1, 17, 600, 2100], [1] * 4, 8, 2, 128, kv_dtype="i8")
    ntok = int(base.tok_base[-1] + base.seq_lens[-1])
    hd = base.num_kv_heads * base.head_dim
    K = workloads.normal_f32(base.seed, workloads.TAG_K, 0, ntok * hd).view(ntok, base.num_kv_heads, -1)
    V = workloads.normal_f32(base.seed, workloads.TAG_V, 0, ntok * hd).view(ntok, base.num_kv_heads, -1)
    Q = workloads.normal_f32(base.seed, workloads.TAG_Q, 0, base.total_q * base.num_q_heads * base.head_dim) * f
    case = workloads.ExplicitCase.wrap(dataclasses.replace(base, softmax_scale=base.softmax_scale / f), K, V,
                                       Q.view(base.total_q, base.num_q_heads, -1))
    q = case.q()
    assert (float(q.abs().max()) > 65504.0) if log2f > 0 else True
    assert (float(q.abs().max()) < 2.0 ** -14) if log2f < 0 else True
    ref = expected_outputs(case)
    for part in (0, 512):
        out = _decode_gpu(case, partition_size=part)
        assert_close(out, ref, "bf16", f"q x 2^{log2f} P={part}")


# ---------------------------------------------------------------- entries without a block
def _with_holes(case, holes):
    t = case.block_tables.copy()
    for s, cols in holes.items():
        for c in cols:
            t[s, c] = -1 if c % 2 == 0 else case.num_blocks + 7
    return dataclasses.replace(case, block_tables=t)


@pytest.mark.parametrize("part", [0, 16, 512])
@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_decode_entries_without_a_block_hold_no_keys(kv, part):
    """Table entries of -1 (or past the pool) inside the visible range hold no
    keys; a sequence that loses every block gets a zero row -- also when its
    keys span several partitions, whose merge then sees no key at all."""
    lens = [100, 40, 33, 16, 600, 1100]
    case = workloads.make_case("holes", 111, lens, [1] * len(lens), 8, 2, 128, kv_dtype=kv)
    nblk = -(-np.asarray(lens) // 16)
    holes = {0: [1, 3], 1: [0], 2: [2], 3: [0], 4: list(range(int(nblk[4]))), 5: list(range(10, 40))}
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "all")
    cache = build_cache(case)
    hc = _with_holes(case, holes)
    out = run_decode(hc, pools, dev, partition_size=part)
    torch.cuda.synchronize()
    ref = expected_outputs(hc, cache=cache)
    assert (ref[3] == 0).all() and (ref[4] == 0).all()
    assert (out[3] == 0).all() and (out[4] == 0).all()
    assert_close(out, ref, "bf16", f"{kv} P={part}")


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_prefill_entries_without_a_block_hold_no_keys(kv):
    lens, new = [100, 40, 300, 16], [30, 40, 100, 16]
    case = workloads.make_case("holes-pf", 112, lens, new, 8, 2, 128, kv_dtype=kv, kind="prefill")
    holes = {0: [1, 3], 1: [0], 2: [2, 5, 6, 7, 8], 3: [0]}
    dev = device()
    pools = alloc_pools(case, dev)
    write_tokens(case, pools, dev, "all")
    cache = build_cache(case)
    hc = _with_holes(case, holes)
    out = run_prefill(hc, pools, dev)
    torch.cuda.synchronize()
    ref = expected_outputs(hc, cache=cache)
    cu = case.cu_q_lens
    assert (out[cu[3]:cu[4]] == 0).all()
    assert_close(out, ref, "bf16", kv)
