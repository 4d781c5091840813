"""The C ABI loads on a machine without a GPU, exports every function that
include/pagedkv.h declares, and rejects invalid host-visible arguments with
the documented status before anything touches a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE = 0, 1, 2, 3
F32, BF16, I8 = 1, 2, 4


def declared_functions(header=HEADER):
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import paged_kv_cache_235_amd as pkv
    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_cache_235_amd import _build
        _build.build()
    return pkv.load_library()


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("kv_cache_write", "paged_attention_decode", "paged_attention_prefill_chunk",
              "paged_attention_decode_workspace_size", "pkv_last_error"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    import paged_kv_cache_235_amd as pkv
    names = declared_functions()
    assert sorted(pkv.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def _desc(nb=8, bs=16, hkv=2, d=128, dt=BF16):
    import paged_kv_cache_235_amd as pkv
    return pkv.CacheDesc(nb, bs, hkv, d, dt)


FAKE = ctypes.c_void_p(0x1000)          # never dereferenced: every call below fails validation


def _decode(lib, desc, **kw):
    a = dict(q=FAKE, q_dtype=BF16, out=FAKE, out_dtype=F32, num_seqs=2, hq=4, k=FAKE, v=FAKE, ks=None, vs=None,
             tables=FAKE, maxb=4, offs=None, lens=FAKE, scale=0.1, window=0, part=0, ws=None, wsb=0)
    a.update(kw)
    return lib.paged_attention_decode(ctypes.byref(desc), a["q"], a["q_dtype"], a["out"], a["out_dtype"],
                                      a["num_seqs"], a["hq"], a["k"], a["v"], a["ks"], a["vs"], a["tables"],
                                      a["maxb"], a["offs"], a["lens"], a["scale"], a["window"], a["part"], a["ws"],
                                      a["wsb"], None)


def test_decode_validation(lib):
    assert _decode(lib, _desc(), num_seqs=0) == PKV_OK                  # no-op
    assert _decode(lib, _desc(), hq=3) == PKV_EINVAL                     # Hq % Hkv
    assert _decode(lib, _desc(d=96)) == PKV_EUNSUPPORTED
    assert _decode(lib, _desc(bs=32)) == PKV_EUNSUPPORTED
    assert _decode(lib, _desc(dt=0)) == PKV_EINVAL
    assert _decode(lib, _desc(nb=0)) == PKV_EINVAL
    assert _decode(lib, _desc(), q_dtype=F32) == PKV_EUNSUPPORTED       # f32 q on a bf16 pool
    assert _decode(lib, _desc(), out_dtype=I8) == PKV_EUNSUPPORTED
    assert _decode(lib, _desc(dt=I8)) == PKV_EINVAL                      # INT8 without scales
    assert _decode(lib, _desc(), ks=FAKE, vs=FAKE) == PKV_EINVAL         # scales on a bf16 pool
    assert _decode(lib, _desc(), part=24) == PKV_EINVAL                  # not a block multiple
    assert _decode(lib, _desc(), window=-1) == PKV_EINVAL
    assert _decode(lib, _desc(), scale=float("nan")) == PKV_EINVAL
    assert _decode(lib, _desc(), scale=-1.0) == PKV_EINVAL
    assert _decode(lib, _desc(), q=None) == PKV_EINVAL
    assert _decode(lib, _desc(), q=ctypes.c_void_p(0x1008)) == PKV_EINVAL   # misaligned
    assert _decode(lib, _desc(), maxb=4, part=16) == PKV_EWORKSPACE      # 4 partitions need scratch
    assert b"workspace" in lib.pkv_last_error()
    assert _decode(lib, _desc(), maxb=4, part=16, ws=ctypes.c_void_p(0x1010), wsb=1 << 20) == PKV_EINVAL  # misaligned
    # offset rows: one row-wide partition may straddle two, so scratch is needed
    assert _decode(lib, _desc(), maxb=4, part=64, offs=FAKE) == PKV_EWORKSPACE


def test_workspace_size(lib):
    f = lib.paged_attention_decode_workspace_size
    assert f(8, 32, 128, 256, 16, 0, 0) == 0                # single pass
    assert f(8, 32, 128, 32, 16, 512, 0) == 0               # one partition covers everything
    assert f(8, 32, 128, 32, 16, 512, 1) > 0                # ... unless offset rows straddle two
    n = f(256, 32, 128, 2048, 16, 512, 0)
    slots = 256 * 32 * 64
    assert n >= slots * (128 + 2) * 4 and n < slots * (128 + 2) * 4 + 512
    assert f(256, 32, 128, 2048, 16, 512, 1) > n            # one more partition per (sequence, head)
    assert f(-1, 32, 128, 2048, 16, 512, 0) == 0


def test_write_validation(lib):
    w = lib.kv_cache_write
    d = _desc()
    assert w(ctypes.byref(d), FAKE, FAKE, BF16, 256, FAKE, 0, FAKE, FAKE, None, None, None) == PKV_OK
    assert w(ctypes.byref(d), FAKE, FAKE, F32, 256, FAKE, 4, FAKE, FAKE, None, None, None) == PKV_EUNSUPPORTED
    assert w(ctypes.byref(d), FAKE, FAKE, BF16, 100, FAKE, 4, FAKE, FAKE, None, None, None) == PKV_EINVAL
    assert w(ctypes.byref(d), FAKE, FAKE, BF16, 260, FAKE, 4, FAKE, FAKE, None, None, None) == PKV_EINVAL
    assert w(ctypes.byref(d), FAKE, FAKE, BF16, 256, FAKE, -1, FAKE, FAKE, None, None, None) == PKV_EINVAL
    d8 = _desc(dt=I8)
    assert w(ctypes.byref(d8), FAKE, FAKE, BF16, 256, FAKE, 4, FAKE, FAKE, None, None, None) == PKV_EINVAL
    assert w(ctypes.byref(d8), FAKE, FAKE, I8, 256, FAKE, 4, FAKE, FAKE, FAKE, FAKE, None) == PKV_EUNSUPPORTED
    assert w(None, FAKE, FAKE, BF16, 256, FAKE, 4, FAKE, FAKE, None, None, None) == PKV_EINVAL


def test_prefill_validation(lib):
    p = lib.paged_attention_prefill_chunk
    d = _desc()
    args = lambda **k: (ctypes.byref(k.get("desc", d)), FAKE, k.get("qd", BF16), FAKE, F32, FAKE,
                        k.get("b", 2), k.get("mq", 16), k.get("hq", 8), FAKE, FAKE, k.get("ks"), k.get("vs"),
                        FAKE, 4, None, FAKE, 0.1, k.get("w", 0), None)
    assert p(*args(b=0)) == PKV_OK
    assert p(*args(mq=0)) == PKV_OK
    assert p(*args(qd=F32)) == PKV_EUNSUPPORTED
    assert p(*args(desc=_desc(dt=F32))) == PKV_EUNSUPPORTED
    assert p(*args(hq=5)) == PKV_EINVAL
    assert p(*args(w=-3)) == PKV_EINVAL
    # INT8 pools need both scale pools; other pools take none
    assert p(*args(desc=_desc(dt=I8))) == PKV_EINVAL
    assert p(*args(desc=_desc(dt=I8), ks=FAKE)) == PKV_EINVAL
    assert p(*args(desc=_desc(dt=I8), ks=FAKE, vs=FAKE, b=0)) == PKV_OK
    assert p(*args(ks=FAKE, vs=FAKE)) == PKV_EINVAL


def test_version(lib):
    assert b"gfx950" in lib.pkv_version()


def test_slot_mapping_validation(lib):
    f = lib.pkv_build_slot_mapping
    d = _desc()
    args = lambda **k: (ctypes.byref(k.get("desc", d)), k.get("cu", FAKE), k.get("b", 2), k.get("lens", FAKE),
                        k.get("tables", FAKE), k.get("maxb", 4), None, k.get("out", FAKE), k.get("rows", 10), None)
    assert f(*args(b=0)) == PKV_OK                       # nothing to do: no launch
    assert f(*args(rows=0)) == PKV_OK
    assert f(*args(b=-1)) == PKV_EINVAL
    assert f(*args(rows=-5)) == PKV_EINVAL
    assert f(*args(maxb=0)) == PKV_EINVAL
    assert f(*args(cu=None)) == PKV_EINVAL
    assert f(*args(out=None)) == PKV_EINVAL
    assert f(*args(desc=_desc(bs=32))) == PKV_EUNSUPPORTED
    assert f(None, FAKE, 2, FAKE, FAKE, 4, None, FAKE, 10, None) == PKV_EINVAL
    assert lib.pkv_last_error()                          # the reason is reported


def test_copy_blocks_validation(lib):
    f = lib.kv_cache_copy_blocks
    d = _desc()
    d8 = _desc(dt=I8)
    args = lambda **k: (ctypes.byref(k.get("desc", d)), k.get("k", FAKE), k.get("v", FAKE), k.get("ks"),
                        k.get("vs"), k.get("src", FAKE), k.get("dst", FAKE), k.get("n", 3), None)
    assert f(*args(n=0)) == PKV_OK
    assert f(*args(n=-1)) == PKV_EINVAL
    assert f(*args(src=None)) == PKV_EINVAL
    assert f(*args(k=ctypes.c_void_p(0x1008))) == PKV_EINVAL          # pools 16-byte aligned
    assert f(*args(ks=FAKE, vs=FAKE)) == PKV_EINVAL                    # no scales for bf16 pools
    assert f(*args(desc=d8)) == PKV_EINVAL                             # INT8 needs both scale pools
    assert f(*args(desc=d8, ks=FAKE)) == PKV_EINVAL
    assert f(*args(desc=d8, ks=FAKE, vs=FAKE, n=0)) == PKV_OK
    assert f(*args(desc=_desc(d=96))) == PKV_EUNSUPPORTED


def test_allocator_abi_rejects_null_and_bad_sizes(lib):
    P = ctypes.c_void_p
    h = P()
    assert lib.pkv_allocator_create(0, 16, ctypes.byref(h)) == PKV_EINVAL and not h.value
    assert lib.pkv_allocator_create(4, 16, None) == PKV_EINVAL
    assert lib.pkv_allocator_create(4, 16, ctypes.byref(h)) == PKV_OK and h.value
    try:
        assert lib.pkv_allocator_num_free(h) == 4
        assert lib.pkv_allocator_num_free(None) == -1
        assert lib.pkv_allocator_refcount(h, 4) == -1 and lib.pkv_allocator_refcount(h, -1) == -1
        ids = (ctypes.c_int32 * 8)()
        assert lib.pkv_allocator_alloc(h, 5, ids) == 5                 # PKV_ENOSPACE
        assert lib.pkv_allocator_num_free(h) == 4
        assert lib.pkv_allocator_alloc(h, -1, ids) == PKV_EINVAL
        assert lib.pkv_allocator_alloc(h, 2, None) == PKV_EINVAL
        n = ctypes.c_int32(0)
        assert lib.pkv_seq_append(h, ids, 8, -1, 1, ids, ids, ctypes.byref(n)) == PKV_EINVAL
        assert lib.pkv_seq_append(None, ids, 8, 0, 1, ids, ids, ctypes.byref(n)) == PKV_EINVAL
        assert lib.pkv_seq_evict_window(h, ids, 10, 0, None) == PKV_EINVAL
        assert lib.pkv_seq_truncate(h, ids, 3, 4) == PKV_EINVAL
    finally:
        assert lib.pkv_allocator_destroy(h) == PKV_OK
    assert lib.pkv_allocator_destroy(None) == PKV_OK


def test_probe_library_exports_its_header_and_rejects_bad_arguments():
    """The measurement kernels (include/pkv_probe.h) live in a library of their
    own; bad arguments are refused before any launch."""
    from paged_kv_cache_235_amd import _build
    if not os.path.exists(_build.PROBE_LIB_PATH):
        _build.build()
    plib = ctypes.CDLL(_build.PROBE_LIB_PATH)
    names = declared_functions(os.path.join(ROOT, "include", "pkv_probe.h"))
    assert names == ["pkv_probe_mfma_bf16", "pkv_probe_stream_read", "pkv_probe_stream_read_spans"]
    for n in names:
        assert hasattr(plib, n), n
    for sr in (plib.pkv_probe_stream_read, plib.pkv_probe_stream_read_spans):
        sr.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        assert sr(FAKE, 15, FAKE, 1, None) == 1          # not whole 16-byte chunks
        assert sr(FAKE, 0, FAKE, 1, None) == 1
        assert sr(FAKE, 16, FAKE, 0, None) == 1          # empty grid
        assert sr(None, 16, FAKE, 1, None) == 1
        assert sr(ctypes.c_void_p(0x1008), 16, FAKE, 1, None) == 1   # not 16-byte aligned
    mm = plib.pkv_probe_mfma_bf16
    mm.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p]
    assert mm(FAKE, -1, 1, 0, None) == 1
    assert mm(FAKE, 1, 0, 0, None) == 1
    assert mm(None, 1, 1, 0, None) == 1
