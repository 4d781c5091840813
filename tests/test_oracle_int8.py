"""Pins of the oracle's INT8 quantiser and of its cache write.

Rule (MicroGen, Key Features: dynamic vector-scale INT8 KV quantisation):
scale = fp16_rne(absmax / 127), code = clamp(rne(x / scale), -127, 127),
binary32 divisions.  Pinned by hand-worked vectors (tests/golden), and by
properties any correct symmetric absmax quantiser has."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.cases import build_cache, to_numpy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_vectors.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_vectors(case):
    q, s = oracle.quantize_vector(np.array(case["x"], np.float32))
    assert s == case["scale_bits"]
    assert q.tolist() == case["codes"]


def _vectors(n=2000, d=128, seed=11):
    x = workloads.normal_f32(seed, workloads.TAG_MISC, 0, n * d).view(n, d)
    out = workloads.bernoulli_mask(seed, workloads.TAG_K_OUTLIER, 0, n * d, 0.01).view(n, d)
    x = torch.where(out, x * 8, x)
    # magnitudes 2^-8 .. 2^11 keep absmax/127 inside fp16's normal range
    mags = torch.exp2(torch.arange(n) % 20 - 8.0).view(n, 1)
    return (x * mags).numpy().astype(np.float32)


def test_quantiser_properties():
    xs = _vectors()
    for x in xs:
        q, s = oracle.quantize_vector(x)
        scale = oracle.f16_to_f64(np.array([s], np.uint16))[0]
        a = np.abs(x).max()
        assert scale > 0
        # the stored scale is the fp16 value nearest absmax/127: within half an fp16 ulp
        assert abs(scale - a / 127.0) <= scale * 2.0 ** -11 * 1.0001
        assert np.all(np.abs(q.astype(int)) <= 127)
        # the largest-magnitude entry lands on +-127
        i = int(np.argmax(np.abs(x)))
        assert q[i] == (127 if x[i] > 0 else -127)
        # signs agree (or the code is zero) and every code is the nearest level
        assert np.all((np.sign(q) == np.sign(x)) | (q == 0))
        err = np.abs(x.astype(np.float64) - q.astype(np.float64) * scale)
        assert np.all(err <= 0.5 * scale * (1 + 1e-6))


def test_quantiser_is_scale_equivariant_by_powers_of_two():
    # multiplying by 2^k (no fp16 range edge crossed) multiplies the scale by 2^k and keeps the codes
    for x in _vectors(200, 64, seed=5)[::3]:
        x = x / np.abs(x).max()
        q0, s0 = oracle.quantize_vector(x)
        q1, s1 = oracle.quantize_vector(x * np.float32(8.0))
        assert np.array_equal(q0, q1)
        assert oracle.f16_to_f64(np.array([s1], np.uint16))[0] == 8 * oracle.f16_to_f64(np.array([s0], np.uint16))[0]


def _small_case(kv_dtype, in_dtype="bf16"):
    return workloads.make_case("write", 21, [5, 17, 32, 1], [5, 17, 32, 1], 4, 2, 64,
                               in_dtype=in_dtype, kv_dtype=kv_dtype, num_blocks=12)


@pytest.mark.parametrize("kv_dtype,in_dtype", [("bf16", "bf16"), ("f32", "f32")])
def test_copy_write_places_every_vector_once_and_keeps_poison(kv_dtype, in_dtype):
    case = _small_case(kv_dtype, in_dtype)
    cache = build_cache(case)
    bs = case.block_size
    written = np.zeros((case.num_blocks, bs), bool)
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        k = to_numpy(case.kv("k", s, 0, L))
        v = to_numpy(case.kv("v", s, 0, L))
        for p in range(L):
            blk = case.block_tables[s, p // bs]
            # the slot of position p is the table entry of its logical block, offset p mod bs
            assert np.array_equal(cache.k[blk, :, p % bs, :], k[p])
            assert np.array_equal(cache.v[blk, :, p % bs, :], v[p])
            assert not written[blk, p % bs]
            written[blk, p % bs] = True
    # every slot nobody wrote still holds the NaN poison
    poison_k = cache.k.transpose(0, 2, 1, 3)[~written]
    if kv_dtype == "f32":
        assert np.isnan(poison_k).all()
    else:
        assert (poison_k == 0x7FC0).all()


def test_negative_slots_are_skipped():
    cache = oracle.Cache(4, 16, 2, 64, "bf16")
    k = np.arange(3 * 2 * 64, dtype=np.uint16).reshape(3, 2, 64)
    cache.write(k, k, "bf16", np.array([-1, 5, -7], np.int32))
    assert np.array_equal(cache.k[0, :, 5, :], k[1])
    cache.k[0, :, 5, :] = 0x7FC0
    assert (cache.k == 0x7FC0).all()


def test_int8_write_stores_the_quantised_vectors():
    case = _small_case("i8")
    cache = build_cache(case)
    bs = case.block_size
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        k = case.kv("k", s, 0, L).float().numpy()
        for p in range(L):
            blk = case.block_tables[s, p // bs]
            for h in range(case.num_kv_heads):
                q, sc = oracle.quantize_vector(k[p, h])
                assert np.array_equal(cache.k[blk, h, p % bs], q)
                assert cache.k_scale[blk, h, p % bs] == sc


def test_int8_write_is_about_half_the_bf16_bytes():
    # INT8 codes plus one fp16 scale per vector: (D + 2) bytes against 2 D for bf16
    for d, ratio in ((128, 256 / 130), (64, 128 / 66)):
        c8 = oracle.Cache(3, 16, 2, d, "i8")
        c16 = oracle.Cache(3, 16, 2, d, "bf16")
        b8 = c8.k.nbytes + c8.k_scale.nbytes
        assert c16.k.nbytes / b8 == pytest.approx(ratio)
