"""ctypes binding of libpagedkv (include/pagedkv.h) for torch tensors.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity) and passed as device pointers together with torch's current HIP
stream; every step of the computation runs in the library's kernels.  There
is no fallback: if ``libpagedkv.so`` is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedkv.so")

PKV_F32, PKV_BF16, PKV_I8 = 1, 2, 4
_TORCH_TO_PKV = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.int8: PKV_I8}
STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE", 4: "PKV_EHIP",
          5: "PKV_ENOSPACE"}

# every symbol include/pagedkv.h declares
EXPORTS = ("kv_cache_write", "paged_attention_decode_workspace_size", "paged_attention_decode",
           "paged_attention_prefill_chunk", "pkv_last_error", "pkv_version",
           "pkv_profile_set_decode_split_event", "pkv_profile_set_decode_start_event",
           "pkv_build_slot_mapping", "kv_cache_copy_blocks", "pkv_allocator_create", "pkv_allocator_destroy",
           "pkv_allocator_num_free", "pkv_allocator_refcount", "pkv_allocator_alloc", "pkv_allocator_retain",
           "pkv_allocator_release", "pkv_seq_append", "pkv_seq_fork", "pkv_seq_truncate",
           "pkv_seq_evict_window", "pkv_seq_compact", "paged_attention_decode_noalloc",
           "paged_attention_decode_noalloc_max_scratch")


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libpagedkv (once).  Raises if it has not been built.  The
    environment variable PKV_LIBRARY names another build of the same library
    (the sanitizer run of the CPU tests uses one)."""
    global _lib
    path = path or os.environ.get("PKV_LIBRARY") or LIB_PATH
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise ImportError(f"{path} is missing: build it with `python -m paged_kv_cache_235_amd._build` "
                                  "(or __graft_entry__.build()); there is no fallback implementation")
            lib = ctypes.CDLL(path)
            P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
            D = ctypes.POINTER(CacheDesc)
            lib.kv_cache_write.restype = ctypes.c_int
            lib.kv_cache_write.argtypes = [D, P, P, i32, i64, P, i32, P, P, P, P, P]
            lib.paged_attention_decode_workspace_size.restype = ctypes.c_size_t
            lib.paged_attention_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
            lib.paged_attention_decode.restype = ctypes.c_int
            lib.paged_attention_decode.argtypes = [D, P, i32, P, i32, i32, i32, P, P, P, P, P, i32, P, P,
                                                   f32, i32, i32, P, ctypes.c_size_t, P]
            lib.paged_attention_decode_noalloc.restype = ctypes.c_int
            lib.paged_attention_decode_noalloc.argtypes = [D, P, i32, P, i32, i32, i32, P, P, P, P, P, i32, P, P,
                                                           f32, i32, i32, P]
            lib.paged_attention_decode_noalloc_max_scratch.restype = ctypes.c_size_t
            lib.paged_attention_decode_noalloc_max_scratch.argtypes = []
            lib.paged_attention_prefill_chunk.restype = ctypes.c_int
            lib.paged_attention_prefill_chunk.argtypes = [D, P, i32, P, i32, P, i32, i32, i32, P, P, P, P, P,
                                                          i32, P, P, f32, i32, P]
            lib.pkv_last_error.restype = ctypes.c_char_p
            lib.pkv_last_error.argtypes = []
            lib.pkv_version.restype = ctypes.c_char_p
            lib.pkv_version.argtypes = []
            lib.pkv_profile_set_decode_split_event.restype = ctypes.c_int
            lib.pkv_profile_set_decode_split_event.argtypes = [P]
            lib.pkv_profile_set_decode_start_event.restype = ctypes.c_int
            lib.pkv_profile_set_decode_start_event.argtypes = [P]
            lib.pkv_build_slot_mapping.restype = ctypes.c_int
            lib.pkv_build_slot_mapping.argtypes = [D, P, i32, P, P, i32, P, P, i32, P]
            lib.kv_cache_copy_blocks.restype = ctypes.c_int
            lib.kv_cache_copy_blocks.argtypes = [D, P, P, P, P, P, P, i32, P]
            lib.pkv_allocator_create.restype = ctypes.c_int
            lib.pkv_allocator_create.argtypes = [i32, i32, ctypes.POINTER(P)]
            lib.pkv_allocator_destroy.restype = ctypes.c_int
            lib.pkv_allocator_destroy.argtypes = [P]
            lib.pkv_allocator_num_free.restype = i32
            lib.pkv_allocator_num_free.argtypes = [P]
            lib.pkv_allocator_refcount.restype = i32
            lib.pkv_allocator_refcount.argtypes = [P, i32]
            for name in ("pkv_allocator_alloc",):
                getattr(lib, name).restype = ctypes.c_int
                getattr(lib, name).argtypes = [P, i32, P]
            for name in ("pkv_allocator_retain", "pkv_allocator_release"):
                getattr(lib, name).restype = ctypes.c_int
                getattr(lib, name).argtypes = [P, P, i32]
            lib.pkv_seq_append.restype = ctypes.c_int
            lib.pkv_seq_append.argtypes = [P, P, i32, i32, i32, P, P, P]
            lib.pkv_seq_fork.restype = ctypes.c_int
            lib.pkv_seq_fork.argtypes = [P, P, i32, P, i32]
            lib.pkv_seq_truncate.restype = ctypes.c_int
            lib.pkv_seq_truncate.argtypes = [P, P, i32, i32]
            lib.pkv_seq_evict_window.restype = ctypes.c_int
            lib.pkv_seq_evict_window.argtypes = [P, P, i32, i32, P]
            lib.pkv_seq_compact.restype = ctypes.c_int
            lib.pkv_seq_compact.argtypes = [P, i32, P]
            _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise PagedKVError(status, load_library().pkv_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype(t: torch.Tensor, what: str) -> int:
    try:
        return _TORCH_TO_PKV[t.dtype]
    except KeyError:
        raise TypeError(f"{what}: unsupported dtype {t.dtype}") from None


def _on_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one GPU")
    return dev


def _contig(t, what):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def cache_desc(k_pool: torch.Tensor) -> CacheDesc:
    """Descriptor of a pool shaped [num_blocks][num_kv_heads][block_size][head_dim]."""
    if k_pool.dim() != 4:
        raise ValueError("pools are [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, hkv, bs, d = k_pool.shape
    return CacheDesc(nb, bs, hkv, d, _dtype(k_pool, "pool"))


def _check_pools(k_pool, v_pool, k_scale, v_scale):
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool differ in shape or dtype")
    _contig(k_pool, "k_pool")
    _contig(v_pool, "v_pool")
    if k_pool.dtype == torch.int8:
        if k_scale is None or v_scale is None:
            raise ValueError("INT8 pools need k_scale and v_scale")
        for sc in (k_scale, v_scale):
            if sc.shape != k_pool.shape[:3] or sc.dtype not in (torch.float16, torch.int16):
                raise ValueError("scale pools are fp16 [num_blocks][num_kv_heads][block_size]")
            _contig(sc, "scale pool")


def kv_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   k_pool: torch.Tensor, v_pool: torch.Tensor,
                   k_scale: torch.Tensor | None = None, v_scale: torch.Tensor | None = None) -> None:
    """Store k, v ([T][Hkv][D], token stride may exceed Hkv*D) into their slots."""
    dev = _on_gpu(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale)
    _check_pools(k_pool, v_pool, k_scale, v_scale)
    desc = cache_desc(k_pool)
    if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must both be [num_tokens][num_kv_heads][head_dim] with equal strides")
    if k.stride(2) != 1 or k.stride(1) != k.shape[2]:
        raise ValueError("each token's heads must be dense (stride only between tokens)")
    if slot_mapping.dtype != torch.int32 or slot_mapping.dim() != 1 or slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("slot_mapping must be int32 [num_tokens]")
    _contig(slot_mapping, "slot_mapping")
    stride = k.stride(0) if k.shape[0] > 1 else k.shape[1] * k.shape[2]
    lib = load_library()
    _check(lib.kv_cache_write(ctypes.byref(desc), _ptr(k), _ptr(v), _dtype(k, "k"), stride,
                              _ptr(slot_mapping), k.shape[0], _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                              _ptr(v_scale), _stream(dev)))


def decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int, max_blocks_per_seq: int,
                          block_size: int = 16, partition_size: int = 512, with_table_offsets: bool = False) -> int:
    return int(load_library().paged_attention_decode_workspace_size(
        num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size, partition_size, int(bool(with_table_offsets))))


def decode_workspace(num_seqs: int, num_q_heads: int, head_dim: int, max_blocks_per_seq: int,
                     block_size: int = 16, partition_size: int = 512, with_table_offsets: bool = False,
                     device=None) -> torch.Tensor:
    """A decode workspace ready for its first call: at least 256 bytes, all zero
    (the work counter in its first bytes must start at zero; each call leaves it
    at zero again)."""
    n = decode_workspace_size(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size, partition_size,
                              with_table_offsets)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _offsets(t, b, what="table_offsets"):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.shape != (b,):
        raise ValueError(f"{what} must be int32 [num_seqs]")
    _contig(t, what)
    return t


def _decode_operands(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, out_dtype,
                     workspace, table_offsets):
    dev = _on_gpu(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, workspace, table_offsets)
    _check_pools(k_pool, v_pool, k_scale, v_scale)
    desc = cache_desc(k_pool)
    _contig(q, "q")
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [num_seqs][num_q_heads][head_dim]")
    b, hq, d = q.shape
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be int32 [num_seqs][max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (b,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    _contig(block_tables, "block_tables")
    _contig(context_lens, "context_lens")
    if out is None:
        out = torch.empty((b, hq, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _contig(out, "out")
    maxb = max(block_tables.shape[1], 1)
    table_offsets = _offsets(table_offsets, b)
    return dev, desc, b, hq, d, out, maxb, table_offsets


def paged_attention_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, softmax_scale: float,
                           sliding_window: int = 0, partition_size: int = 512,
                           k_scale: torch.Tensor | None = None, v_scale: torch.Tensor | None = None,
                           out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                           workspace: torch.Tensor | None = None,
                           table_offsets: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention for q [num_seqs][Hq][D]; returns out [num_seqs][Hq][D]."""
    dev, desc, b, hq, d, out, maxb, table_offsets = _decode_operands(
        q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, out_dtype, workspace, table_offsets)
    need = decode_workspace_size(b, hq, d, maxb, desc.block_size, partition_size, table_offsets is not None) if b else 0
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        # zeroed: the work counter at its head must start at zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    lib = load_library()
    _check(lib.paged_attention_decode(
        ctypes.byref(desc), _ptr(q), _dtype(q, "q"), _ptr(out), _dtype(out, "out"), b, hq, _ptr(k_pool),
        _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), maxb, _ptr(table_offsets), _ptr(context_lens),
        float(softmax_scale), int(sliding_window), int(partition_size), _ptr(workspace) if need else None,
        need, _stream(dev)))
    return out


def paged_attention_decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor, softmax_scale: float,
                                   sliding_window: int = 0, partition_size: int = 512,
                                   k_scale: torch.Tensor | None = None, v_scale: torch.Tensor | None = None,
                                   out: torch.Tensor = None,
                                   table_offsets: torch.Tensor | None = None) -> torch.Tensor:
    """paged_attention_decode with the library's fixed scratch instead of a
    workspace: the caller passes ``out`` and the library allocates nothing."""
    if out is None:
        raise ValueError("paged_attention_decode_noalloc writes into a caller-provided out")
    dev, desc, b, hq, d, out, maxb, table_offsets = _decode_operands(
        q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, out.dtype, None, table_offsets)
    lib = load_library()
    _check(lib.paged_attention_decode_noalloc(
        ctypes.byref(desc), _ptr(q), _dtype(q, "q"), _ptr(out), _dtype(out, "out"), b, hq, _ptr(k_pool),
        _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), maxb, _ptr(table_offsets), _ptr(context_lens),
        float(softmax_scale), int(sliding_window), int(partition_size), _stream(dev)))
    return out


def decode_noalloc_max_scratch() -> int:
    """Bytes of the fixed scratch the allocation-free decode uses on each GPU."""
    return int(load_library().paged_attention_decode_noalloc_max_scratch())


def paged_attention_prefill_chunk(q: torch.Tensor, cu_q_lens: torch.Tensor, seq_lens: torch.Tensor,
                                  k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                                  max_q_len: int, softmax_scale: float, sliding_window: int = 0,
                                  out: torch.Tensor | None = None,
                                  out_dtype: torch.dtype = torch.float32,
                                  k_scale: torch.Tensor | None = None,
                                  v_scale: torch.Tensor | None = None,
                                  table_offsets: torch.Tensor | None = None) -> torch.Tensor:
    """Chunked-prefill attention for q [total_rows][Hq][D] (bf16) over bf16 or INT8 pools."""
    dev = _on_gpu(q, cu_q_lens, seq_lens, k_pool, v_pool, block_tables, out, k_scale, v_scale, table_offsets)
    _check_pools(k_pool, v_pool, k_scale, v_scale)
    desc = cache_desc(k_pool)
    _contig(q, "q")
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [total_rows][num_q_heads][head_dim]")
    b = seq_lens.shape[0]
    if cu_q_lens.dtype != torch.int32 or cu_q_lens.shape != (b + 1,):
        raise ValueError("cu_q_lens must be int32 [num_seqs + 1]")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be int32 [num_seqs]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be int32 [num_seqs][max_blocks_per_seq]")
    for t, n in ((cu_q_lens, "cu_q_lens"), (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        _contig(t, n)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _contig(out, "out")
    lib = load_library()
    _check(lib.paged_attention_prefill_chunk(
        ctypes.byref(desc), _ptr(q), _dtype(q, "q"), _ptr(out), _dtype(out, "out"), _ptr(cu_q_lens), b,
        int(max_q_len), q.shape[1], _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
        max(block_tables.shape[1], 1), _ptr(_offsets(table_offsets, b)), _ptr(seq_lens), float(softmax_scale),
        int(sliding_window), _stream(dev)))
    return out


def build_slot_mapping(cu_q_lens: torch.Tensor, seq_lens: torch.Tensor, block_tables: torch.Tensor,
                       k_pool: torch.Tensor, out: torch.Tensor | None = None,
                       total_rows: int | None = None, table_offsets: torch.Tensor | None = None) -> torch.Tensor:
    """Slot of every new row (row i of sequence s at position seq_lens[s] - C_s + i),
    computed on the GPU from the block tables; -1 where the table holds no block."""
    dev = _on_gpu(cu_q_lens, seq_lens, block_tables, out)
    desc = cache_desc(k_pool)
    b = seq_lens.shape[0]
    for t, n in ((cu_q_lens, "cu_q_lens"), (seq_lens, "seq_lens"), (block_tables, "block_tables")):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
        _contig(t, n)
    if cu_q_lens.shape != (b + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("cu_q_lens must be [num_seqs + 1] and block_tables [num_seqs][max_blocks]")
    if out is None:
        if total_rows is None:
            total_rows = int(cu_q_lens[-1].item()) if b else 0
        out = torch.empty(total_rows, dtype=torch.int32, device=dev)
    if out.dtype != torch.int32 or out.dim() != 1:
        raise ValueError("out must be int32 [total_rows]")
    _contig(out, "out")
    lib = load_library()
    _check(lib.pkv_build_slot_mapping(ctypes.byref(desc), _ptr(cu_q_lens), b, _ptr(seq_lens), _ptr(block_tables),
                                      max(block_tables.shape[1], 1), _ptr(_offsets(table_offsets, b)), _ptr(out),
                                      out.shape[0], _stream(dev)))
    return out


def kv_cache_copy_blocks(src_blocks: torch.Tensor, dst_blocks: torch.Tensor, k_pool: torch.Tensor,
                         v_pool: torch.Tensor, k_scale: torch.Tensor | None = None,
                         v_scale: torch.Tensor | None = None) -> None:
    """Block dst_blocks[n] of every pool becomes a copy of block src_blocks[n]."""
    dev = _on_gpu(src_blocks, dst_blocks, k_pool, v_pool, k_scale, v_scale)
    _check_pools(k_pool, v_pool, k_scale, v_scale)
    desc = cache_desc(k_pool)
    if (src_blocks.dtype != torch.int32 or dst_blocks.dtype != torch.int32 or src_blocks.dim() != 1
            or src_blocks.shape != dst_blocks.shape):
        raise ValueError("src_blocks and dst_blocks must be int32 [num_pairs]")
    _contig(src_blocks, "src_blocks")
    _contig(dst_blocks, "dst_blocks")
    lib = load_library()
    _check(lib.kv_cache_copy_blocks(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(src_blocks), _ptr(dst_blocks), src_blocks.shape[0], _stream(dev)))


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _row(a, what):
    import numpy as np
    if not isinstance(a, np.ndarray) or a.dtype != np.int32 or a.ndim != 1 or not a.flags.c_contiguous \
            or not a.flags.writeable:
        raise ValueError(f"{what} must be a writeable contiguous numpy int32 vector")
    return a


class BlockAllocator:
    """Host-side owner of a pool's blocks (include/pagedkv.h, pkv_allocator_*):
    O(1) free stack, reference counts for shared blocks, and the table edits of
    appending, forking, rolling back and window eviction.  Table rows are numpy
    int32 vectors (-1 = no block) that the caller copies to the device."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pkv_allocator_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:       # interpreter shutdown: the library may already be gone
            pass

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_allocator_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pkv_allocator_refcount(self._h, int(block)))

    def alloc(self, n: int):
        import numpy as np
        ids = np.empty(max(int(n), 1), np.int32)
        _check(self._lib.pkv_allocator_alloc(self._h, int(n), _np_ptr(ids)))
        return ids[:int(n)]

    def retain(self, ids):
        import numpy as np
        ids = np.ascontiguousarray(ids, np.int32)
        _check(self._lib.pkv_allocator_retain(self._h, _np_ptr(ids), ids.size))

    def release(self, ids):
        import numpy as np
        ids = np.ascontiguousarray(ids, np.int32)
        _check(self._lib.pkv_allocator_release(self._h, _np_ptr(ids), ids.size))

    def append(self, row, length: int, num_new: int):
        """Blocks for num_new tokens after `length`; returns the copy-on-write
        pairs [(src, dst)] to run through kv_cache_copy_blocks first."""
        import numpy as np
        row = _row(row, "row")
        src = np.zeros(1, np.int32)
        dst = np.zeros(1, np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_append(self._h, _np_ptr(row), row.size, int(length), int(num_new),
                                        _np_ptr(src), _np_ptr(dst), ctypes.byref(n)))
        return [(int(src[0]), int(dst[0]))] if n.value else []

    def fork(self, parent_row, length: int, child_row):
        import numpy as np
        parent_row = np.ascontiguousarray(parent_row, np.int32)
        child_row = _row(child_row, "child_row")
        _check(self._lib.pkv_seq_fork(self._h, _np_ptr(parent_row), int(length), _np_ptr(child_row),
                                      child_row.size))

    def truncate(self, row, length: int, new_length: int):
        row = _row(row, "row")
        _check(self._lib.pkv_seq_truncate(self._h, _np_ptr(row), int(length), int(new_length)))

    @staticmethod
    def compact(row, offset: int) -> int:
        """Drop the row's leading released entries; returns the new offset."""
        row = _row(row, "row")
        off = ctypes.c_int32(int(offset))
        _check(load_library().pkv_seq_compact(_np_ptr(row), row.size, ctypes.byref(off)))
        return int(off.value)

    def evict_window(self, row, length: int, window: int) -> int:
        row = _row(row, "row")
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_seq_evict_window(self._h, _np_ptr(row), int(length), int(window), ctypes.byref(n)))
        return int(n.value)


def set_decode_split_event(event) -> None:
    """Profiling aid: record ``event`` (torch.cuda.Event or None) between the
    decode partition and merge kernels of later decode calls on this thread."""
    if event is not None and not event.cuda_event:
        event.record()          # torch creates the HIP event on first record
    ptr = None if event is None else ctypes.c_void_p(event.cuda_event)
    load_library().pkv_profile_set_decode_split_event(ptr)


def set_decode_start_event(event) -> None:
    """Profiling aid: record ``event`` (torch.cuda.Event or None) right before
    the decode partition kernel of later decode calls on this thread."""
    if event is not None and not event.cuda_event:
        event.record()
    ptr = None if event is None else ctypes.c_void_p(event.cuda_event)
    load_library().pkv_profile_set_decode_start_event(ptr)


def last_error() -> str:
    return load_library().pkv_last_error().decode()


def version() -> str:
    return load_library().pkv_version().decode()
