"""Reference implementation (oracle) of attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never loads it and shares no code with it; a missing GPU extension is an
error there, never a reason to come here.

The arithmetic lives in ``pkv_oracle.c`` (plain single-threaded C99, fp64
attention).  This module compiles it with gcc on first use and marshals numpy
arrays through ctypes.  bf16 and fp16 arrays are carried as ``np.uint16`` bit
patterns.  Parity status of every function: pinned by ``tests/test_oracle_*``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "pkv_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, BF16, I8 = 0, 1, 3
DTYPES = {"f32": F32, "bf16": BF16, "i8": I8}
NP_TYPES = {F32: np.float32, BF16: np.uint16, I8: np.int8}

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-o", tmp, SOURCE, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    """The compiled oracle (built on first use).  The environment variable
    PKV_ORACLE_LIBRARY names another build of the same source to load instead
    (the sanitizer run of the CPU tests uses one)."""
    global _lib
    with _lock:
        if _lib is None:
            other = os.environ.get("PKV_ORACLE_LIBRARY")
            if other:
                _lib = _declare(ctypes.CDLL(other))
            else:
                if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
                    build()
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _declare(L):
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [f32]
    L.orc_f16_to_f64.restype = ctypes.c_double
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f64.restype = ctypes.c_double
    L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_f16_array.argtypes = [P, i64, P]
    L.orc_f16_to_f64_array.argtypes = [P, i64, P]
    L.orc_quantize_vector.argtypes = [P, i32, P, P]
    L.orc_kv_write.restype = ctypes.c_int
    L.orc_kv_write.argtypes = [i32, i32, i32, i32, i32, P, P, i32, i64, P, i32, P, P, P, P]
    L.orc_slot_mapping.restype = ctypes.c_int
    L.orc_slot_mapping.argtypes = [i32, i32, i32, P, P, P, i32, P]
    L.orc_copy_blocks.restype = ctypes.c_int
    L.orc_copy_blocks.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i32]
    L.orc_attention.restype = ctypes.c_int
    L.orc_attention.argtypes = [i32, i32, i32, i32, i32, P, i32, i32, i32, P, P, P, P, P, P, P,
                                i32, f32, i32, P, P, i64]
    L.orc_decode.restype = ctypes.c_int
    L.orc_decode.argtypes = [i32, i32, i32, i32, i32, P, i32, i32, i32, P, P, P, P, P, i32, P,
                             f32, i32, P, P, i64]
    L.orc_decode_split.restype = ctypes.c_int
    L.orc_decode_split.argtypes = [i32, i32, i32, i32, i32, P, i32, i32, i32, P, P, P, P, P, i32,
                                   P, f32, i32, i32, P]
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


# ------------------------------------------------------------------ numbers
def f32_to_f16(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_to_f64(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_f16_to_f64_array(_ptr(h), h.size, _ptr(out))
    return out


def bf16_to_f64(b) -> np.ndarray:
    b = _c(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantize_vector(x):
    """(int8 codes, fp16 scale bits) of one vector."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.int8)
    s = np.zeros(1, np.uint16)
    lib().orc_quantize_vector(_ptr(x), x.size, _ptr(q), _ptr(s))
    return q, int(s[0])


# ------------------------------------------------------------------ cache
class Cache:
    """Host pools in the library's layout: [NB][Hkv][bs][D] (+ [NB][Hkv][bs] scales)."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.kv_dtype = DTYPES[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        t = NP_TYPES[self.kv_dtype]
        self.k = np.empty(shape, t)
        self.v = np.empty(shape, t)
        self.k_scale = self.v_scale = None
        if self.kv_dtype == I8:
            self.k_scale = np.empty(shape[:3], np.uint16)
            self.v_scale = np.empty(shape[:3], np.uint16)
        self.poison()

    def poison(self):
        """Fill with NaN (fp32/bf16), -128 codes and NaN scales (INT8)."""
        if self.kv_dtype == F32:
            self.k.fill(np.nan)
            self.v.fill(np.nan)
        elif self.kv_dtype == BF16:
            self.k.fill(0x7FC0)
            self.v.fill(0x7FC0)
        else:
            self.k.fill(-128)
            self.v.fill(-128)
            self.k_scale.fill(0x7E00)
            self.v_scale.fill(0x7E00)

    def desc(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim, self.kv_dtype)

    def write(self, k, v, in_dtype, slots, token_stride=None):
        """Reference cache write of tokens k, v: [T][Hkv][D] (or token_stride apart)."""
        in_dtype = DTYPES[in_dtype] if isinstance(in_dtype, str) else in_dtype
        k = _c(k, NP_TYPES[in_dtype])
        v = _c(v, NP_TYPES[in_dtype])
        slots = _c(slots, np.int32)
        if token_stride is None:
            token_stride = self.num_kv_heads * self.head_dim
        rc = lib().orc_kv_write(*self.desc(), _ptr(k), _ptr(v), in_dtype, token_stride, _ptr(slots),
                                slots.size, _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
                                _ptr(self.v_scale))
        _check(rc, "kv_write")


def logical_tables(block_tables, table_offsets=None) -> np.ndarray:
    """The logical block table of offset rows ("MicroGen", Key Features: window
    eviction): column c of row s holds logical block c + table_offsets[s], so
    logical entry b is row[b - offset] and the blocks before the offset (released)
    are -1.  Without offsets the table is its own logical table."""
    tables = _c(block_tables, np.int32)
    if table_offsets is None:
        return tables
    off = _c(table_offsets, np.int32)
    if tables.ndim != 2 or off.shape != (tables.shape[0],) or (off < 0).any():
        raise ValueError("table_offsets must be non-negative int32 [num_seqs]")
    width = tables.shape[1] + (int(off.max()) if off.size else 0)
    out = np.full((tables.shape[0], max(width, 1)), -1, np.int32)
    for s in range(tables.shape[0]):
        out[s, off[s]:off[s] + tables.shape[1]] = tables[s]
    return out


def slot_mapping(num_blocks, block_size, cu_q_lens, seq_lens, block_tables, table_offsets=None) -> np.ndarray:
    """Reference slot of every new row: row i of sequence s sits at position
    seq_lens[s] - C_s + i; -1 where the table holds no valid block."""
    cu = _c(cu_q_lens, np.int32)
    lens = _c(seq_lens, np.int32)
    tables = logical_tables(block_tables, table_offsets)
    out = np.empty(int(cu[-1]) if cu.size else 0, np.int32)
    rc = lib().orc_slot_mapping(num_blocks, block_size, lens.size, _ptr(cu), _ptr(lens), _ptr(tables),
                                tables.shape[1] if tables.ndim == 2 else 0, _ptr(out))
    _check(rc, "slot_mapping")
    return out


def copy_blocks(cache: "Cache", src, dst) -> None:
    """Reference block copy: block dst[n] of every pool becomes block src[n]."""
    src = _c(src, np.int32)
    dst = _c(dst, np.int32)
    if src.shape != dst.shape:
        raise ValueError("src and dst differ in length")
    rc = lib().orc_copy_blocks(*cache.desc(), _ptr(cache.k), _ptr(cache.v), _ptr(cache.k_scale),
                               _ptr(cache.v_scale), _ptr(src), _ptr(dst), src.size)
    _check(rc, "copy_blocks")


def attention(cache: Cache, q, q_dtype, cu_q_lens, seq_lens, block_tables, softmax_scale,
              window=0, weights=False, table_offsets=None):
    """Reference attention for all query rows; returns out [rows][Hq][D] (and weights)."""
    q_dtype = DTYPES[q_dtype] if isinstance(q_dtype, str) else q_dtype
    q = _c(q, NP_TYPES[q_dtype])
    cu = _c(cu_q_lens, np.int32)
    lens = _c(seq_lens, np.int32)
    tables = logical_tables(block_tables, table_offsets)
    rows, hq, d = q.shape
    out = np.zeros((rows, hq, d), np.float64)
    wstride = int(lens.max()) if lens.size else 0
    w = np.zeros((rows, hq, max(wstride, 1)), np.float64) if weights else None
    rc = lib().orc_attention(*cache.desc(), _ptr(q), q_dtype, lens.size, hq, _ptr(cu), _ptr(lens),
                             _ptr(cache.k), _ptr(cache.v), _ptr(cache.k_scale), _ptr(cache.v_scale),
                             _ptr(tables), tables.shape[1], softmax_scale, window, _ptr(out), _ptr(w),
                             max(wstride, 1))
    _check(rc, "attention")
    return (out, w) if weights else out


def decode(cache: Cache, q, q_dtype, context_lens, block_tables, softmax_scale, window=0,
           weights=False, table_offsets=None):
    """Reference decode: one query per sequence at position context_lens[s] - 1."""
    q_dtype = DTYPES[q_dtype] if isinstance(q_dtype, str) else q_dtype
    q = _c(q, NP_TYPES[q_dtype])
    lens = _c(context_lens, np.int32)
    tables = logical_tables(block_tables, table_offsets)
    b, hq, d = q.shape
    out = np.zeros((b, hq, d), np.float64)
    wstride = max(int(lens.max()) if lens.size else 1, 1)
    w = np.zeros((b, hq, wstride), np.float64) if weights else None
    rc = lib().orc_decode(*cache.desc(), _ptr(q), q_dtype, b, hq, _ptr(cache.k), _ptr(cache.v),
                          _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(tables), tables.shape[1],
                          _ptr(lens), softmax_scale, window, _ptr(out), _ptr(w), wstride)
    _check(rc, "decode")
    return (out, w) if weights else out


def decode_split(cache: Cache, q, q_dtype, context_lens, block_tables, softmax_scale,
                 partition_size, window=0):
    """Reference decode computed per partition and merged (checks the merge algebra)."""
    q_dtype = DTYPES[q_dtype] if isinstance(q_dtype, str) else q_dtype
    q = _c(q, NP_TYPES[q_dtype])
    lens = _c(context_lens, np.int32)
    tables = _c(block_tables, np.int32)
    b, hq, d = q.shape
    out = np.zeros((b, hq, d), np.float64)
    rc = lib().orc_decode_split(*cache.desc(), _ptr(q), q_dtype, b, hq, _ptr(cache.k), _ptr(cache.v),
                                _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(tables),
                                tables.shape[1], _ptr(lens), softmax_scale, window, partition_size,
                                _ptr(out))
    _check(rc, "decode_split")
    return out
