"""The INT8 cache write's division-free quantiser, checked exhaustively on the CPU.

The write kernel quantises bf16 inputs as rint(x * rcp(sf)) and falls back to
the IEEE division rint(fp32(x / sf)) only when the product lies within 2^-13 of
a half-integer.  The argument for that ("MicroGen", Key Features: dynamic
per-vector INT8 KV; the codes must be the division's codes exactly) rests on
two facts about bf16 numerators and binary16 scales, both checked here over
their whole domain with numpy's IEEE binary32 arithmetic:

* with the scale rounded as the kernel rounds it (sf = binary16(fp32(amax / 127)),
  |x| <= amax), |x| / sf never exceeds 191;
* for every positive binary16 scale, every positive bf16 x with
  1/8 <= x / sf <= 191, and every reciprocal within 1 ulp of 1/sf (the hardware
  reciprocal's stated accuracy: the correctly rounded value and its two
  neighbours), a product at least 2^-13 from every half-integer rounds to the
  integer the IEEE quotient rounds to.

and, for the scale itself, that binary16(fp32(amax * fp32(1/127))) equals
binary16(fp32(amax / 127)) for every bf16 amax (the kernel's scale of bf16
inputs).

Below x / sf = 1/8 both give 0 (the product is below 1/8 + 2^-20), and negative
x mirror positive x (the product, the quotient and round-half-even are all odd
functions).  This checks the kernel's arithmetic, not the oracle, and calls
neither.
"""
import numpy as np

THRESH = np.float32(0.5 - 2.0 ** -13)


def _bf16_positive():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)          # subnormals .. largest finite
    return (bits << 16).view(np.float32)


def _f16_positive():
    bits = np.arange(0x0001, 0x7C00, dtype=np.uint16)          # subnormals .. 65504
    return bits.view(np.float16).astype(np.float32)


def test_ratio_bound_of_rounded_scales():
    amax = _bf16_positive()
    sf = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16).astype(np.float32)
    live = (sf > 0) & np.isfinite(sf)
    ratio = amax[live] / sf[live]
    assert ratio.max() <= 191.0, ratio.max()
    # the bound is nearly reached: scales rounded up from half the smallest subnormal
    assert ratio.max() > 150.0


def test_product_rounds_like_the_division():
    x = _bf16_positive()
    sfs = _f16_positive()
    lo = np.searchsorted(x, sfs / np.float32(8.0), side="left")
    hi = np.searchsorted(x, sfs * np.float32(191.0), side="right")
    counts = hi - lo
    checked = flagged = 0
    chunk = 2048
    for c0 in range(0, sfs.size, chunk):
        sf_c = sfs[c0:c0 + chunk]
        lo_c, n_c = lo[c0:c0 + chunk], counts[c0:c0 + chunk]
        tot = int(n_c.sum())
        starts = np.repeat(np.cumsum(n_c) - n_c, n_c)
        xi = np.arange(tot) - starts + np.repeat(lo_c, n_c)
        xv = x[xi]
        sv = np.repeat(sf_c, n_c)
        exact = np.rint(xv / sv)                                 # rint of the fp32 quotient
        r0 = np.float32(1.0) / sv
        for r in (np.nextafter(r0, np.float32(0.0)), r0, np.nextafter(r0, np.float32(np.inf))):
            q = xv * r
            c = np.rint(q)
            near = np.abs(q - c) > THRESH
            bad = (~near) & (c != exact)
            assert not bad.any(), (xv[bad][:4], sv[bad][:4])
            checked += tot
            flagged += int(near.sum())
    assert checked > 10_000_000
    # the fallback is the rare case (exact ties and products just beside them)
    assert flagged < checked * 2e-3, (flagged, checked)


def test_exact_ties_take_the_division():
    # x / sf = h exactly for a half-integer h: the product must be flagged for
    # every reciprocal within 1 ulp, whatever side of h it lands on
    sfs = _f16_positive()
    for h in (0.5, 1.5, 2.5, 63.5, 126.5):
        xv = (sfs * np.float32(h)).astype(np.float32)
        keep = ((xv.view(np.uint32) & 0xFFFF) == 0) & (xv / sfs == np.float32(h))   # bf16-exact ties
        xv, sv = xv[keep], sfs[keep]
        assert xv.size > 10
        r0 = np.float32(1.0) / sv
        for r in (np.nextafter(r0, np.float32(0.0)), r0, np.nextafter(r0, np.float32(np.inf))):
            q = xv * r
            assert (np.abs(q - np.rint(q)) > THRESH).all(), h


def test_scale_by_the_reciprocal_of_127():
    # the write kernel takes the scale of bf16 inputs as binary16(fp32(amax * c)),
    # c = fp32(1/127), in place of binary16(fp32(amax / 127)): amax is then a bf16
    # value, and over every one of them (zero and infinity included) the two agree
    bits = np.arange(0x0000, 0x7F81, dtype=np.uint32)             # +0 .. +inf
    amax = (bits << 16).view(np.float32)
    c = np.float32(float.fromhex("0x1.020408p-7"))
    assert c == np.float32(1.0) / np.float32(127.0)
    with np.errstate(over="ignore"):
        by_division = (amax / np.float32(127.0)).astype(np.float16)
        by_product = (amax * c).astype(np.float16)
    assert np.array_equal(by_division.view(np.uint16), by_product.view(np.uint16))
    # the fp32 values themselves differ often: only the binary16 rounding agrees
    assert np.count_nonzero((amax / np.float32(127.0)) != (amax * c)) > 100
