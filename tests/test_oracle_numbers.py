"""Pins of the oracle's number-format conversions against numpy (IEEE 754).

binary16 rounding decides the INT8 scale bytes, so the oracle's own
conversion (written from the IEEE definition) is checked against numpy's
float32 -> float16 cast, which rounds to nearest, ties to even."""
import numpy as np

import oracle


def _all_f16_values():
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    return h, h.view(np.float16)


def test_f16_to_f64_matches_numpy_for_every_code():
    h, f = _all_f16_values()
    got = oracle.f16_to_f64(h)
    ref = f.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_to_f64_matches_numpy_for_every_code():
    lib = oracle.lib()
    codes = np.arange(0x10000, dtype=np.uint32)
    ref = (codes << 16).view(np.float32).astype(np.float64)
    got = np.array([lib.orc_bf16_to_f64(int(c)) for c in codes[::7]])
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])


def _f32_to_f16_cases():
    h, f = _all_f16_values()
    finite = np.isfinite(f)
    vals = f[finite].astype(np.float32)
    pos = np.unique(np.abs(f[finite].astype(np.float64)))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)            # exact ties (representable in f32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    special = np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e6, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 2.0 ** -14,
                        2.0 ** -14 * (1 - 2.0 ** -12), 1e-30, -1e-30], np.float32)
    rng = np.random.default_rng(0)
    rand = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 18, 200000))).astype(np.float32)
    return np.concatenate([vals, mids, -mids, up, dn, -up, special, rand])


def test_f32_to_f16_matches_numpy_rne_including_ties_subnormals_overflow():
    x = _f32_to_f16_cases()
    got = oracle.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


def test_f32_to_f16_ties_go_to_even():
    # 1 + 2^-11 lies halfway between 1 (even fraction) and 1 + 2^-10 (odd)
    assert oracle.f32_to_f16(np.float32(1 + 2.0 ** -11))[()] == 0x3C00
    # 1 + 3 * 2^-11 lies halfway between 1 + 2^-10 (odd) and 1 + 2^-9 (even)
    assert oracle.f32_to_f16(np.float32(1 + 3 * 2.0 ** -11))[()] == 0x3C02
    # 2^-25 is halfway between 0 and the smallest subnormal 2^-24: ties to 0
    assert oracle.f32_to_f16(np.float32(2.0 ** -25))[()] == 0x0000
    # 3 * 2^-25 is halfway between 2^-24 (code 1, odd) and 2^-23 (code 2, even)
    assert oracle.f32_to_f16(np.float32(3 * 2.0 ** -25))[()] == 0x0002
