"""The benchmark's measurement kernels (libconvrot_ceiling.so) compute what
include/convrot_ceiling.h says they do (GPU).

They are not on the hot path, but the benchmark reports rates from them, so
a kernel that skipped work would report a ceiling that is not one: the HBM
stream must write every destination chunk as the XOR of its source planes,
and the MFMA loop must report the operation count its launch performs and
leave one value per lane in the sink.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    L = ctypes.CDLL(os.path.join(ROOT, "hadamard_rotated_int8_amd", "libconvrot_ceiling.so"))
    L.convrot_ceiling_stream.restype = ctypes.c_int32
    L.convrot_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.convrot_ceiling_mfma_i8.restype = ctypes.c_int64
    L.convrot_ceiling_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p]
    return L


@pytest.mark.parametrize("ratio", [1, 2, 4])
@pytest.mark.parametrize("chunks,grid", [(1, 1), (1000, 3), (4096 * 3 + 5, 7), (65536, 512)])
def test_stream_writes_xor_of_planes(ratio, chunks, grid):
    """Every 16-byte destination chunk is the XOR of the ratio source chunks
    at the same index of each plane; sizes that leave a ragged last round
    of the grid-stride loop, and a grid larger than the work."""
    print(f"[gpu] stream ratio={ratio} chunks={chunks} grid={grid}", flush=True)
    L = _lib()
    rng = np.random.default_rng(chunks + ratio)
    words = chunks * 4
    src = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, size=ratio * words, dtype=np.int64)
                           .astype(np.int32)).cuda()
    dst = torch.full((words + 64,), 12345, dtype=torch.int32, device="cuda")  # guard words
    rc = L.convrot_ceiling_stream(src.data_ptr(), dst.data_ptr(), chunks * 16, ratio, grid,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    planes = src.cpu().numpy().reshape(ratio, words)
    want = np.bitwise_xor.reduce(planes, axis=0)
    got = dst.cpu().numpy()
    assert np.array_equal(got[:words], want)
    assert np.all(got[words:] == 12345)  # nothing written past the destination


def test_mfma_loop_reports_its_work():
    """The returned count is grid x 4 waves x iters x 24 MFMAs x 65536 int8
    operations, and every lane of the sink is written."""
    print("[gpu] mfma loop", flush=True)
    L = _lib()
    rng = np.random.default_rng(5)
    a = torch.from_numpy(rng.integers(-127, 128, size=(64, 256), dtype=np.int64)
                         .astype(np.int8)).cuda()
    b = torch.from_numpy(rng.integers(-127, 128, size=(96, 256), dtype=np.int64)
                         .astype(np.int8)).cuda()
    grid, iters = 3, 10
    sink = torch.full((grid * 256 + 64,), 0x7A7A7A7A, dtype=torch.int32, device="cuda")
    ops = L.convrot_ceiling_mfma_i8(a.data_ptr(), 256, 64, b.data_ptr(), 256, 96, iters, grid,
                                    sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert ops == grid * 4 * iters * 24 * 65536
    s = sink.cpu().numpy()
    assert np.all(s[grid * 256:] == 0x7A7A7A7A)  # only grid * 256 lanes written
    assert np.count_nonzero(s[:grid * 256] != 0x7A7A7A7A) > grid * 256 // 2
