"""The streaming-read measurement kernels (include/pkv_probe.h, grid-stride
and contiguous-span orders) read every 16-byte chunk of their buffer exactly once: the XOR of what the threads report
equals the XOR of the whole buffer, for ragged sizes and any grid.  (A chunk
read twice would cancel out of the XOR, one never read would be missing.)"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plib():
    from paged_kv_cache_235_amd import _build
    assert os.path.exists(_build.PROBE_LIB_PATH), "libpkvprobe.so is not built"
    lib = ctypes.CDLL(_build.PROBE_LIB_PATH)
    for f in (lib.pkv_probe_stream_read, lib.pkv_probe_stream_read_spans):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.pkv_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                        ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("order", ["grid_stride", "spans"])
@pytest.mark.parametrize("chunks,grid", [(1, 1), (65537, 3), (1 << 20, 64), (123457, 1000), (5, 8)])
def test_stream_read_covers_every_chunk_once(plib, chunks, grid, order):
    dev = torch.device("cuda", 0)
    words = np.random.default_rng(chunks + grid).integers(0, 2 ** 32, size=4 * chunks, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fn = plib.pkv_probe_stream_read if order == "grid_stride" else plib.pkv_probe_stream_read_spans
    assert fn(ctypes.c_void_p(buf.data_ptr()), 16 * chunks, ctypes.c_void_p(sink.data_ptr()), grid, stream) == 0
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_mfma_probe_runs_and_writes_finite_sums(plib):
    dev = torch.device("cuda", 0)
    sink = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert plib.pkv_probe_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), 10, 4, 1, stream) == 0
    s = sink.cpu()
    assert torch.isfinite(s).all() and (s > 0).any()
