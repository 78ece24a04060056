"""GPU checks of the HBM microbenchmarks (include/moe_micro.h, libmoe_micro.so): every
read kernel folds what it reads into a per-thread XOR, so over all threads the XOR of
the outputs equals the XOR of the 32-bit words the pattern covers, taken once each.
That holds only if each word of the read set is read an odd number of times and no
word outside it is read, which is what the bandwidth figures assume.  The expected
value comes from numpy over the same seeded buffer; the buffers are small, the grids
those of the benchmark's patterns."""

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int


@pytest.fixture(scope="module")
def micro():
    from sparse_moe_expert_route_amd import build as B
    if not os.path.exists(B.MICRO_LIB):
        pytest.fail("libmoe_micro.so is not built")
    L = ctypes.CDLL(B.MICRO_LIB)
    L.moe_micro_hbm_read.argtypes = [vp, sz, vp, i32, i32, vp]
    L.moe_micro_hbm_read_groups.argtypes = [vp, sz, sz, sz, i32, vp, i32, vp]
    return L


def _buffer(nbytes, seed):
    words = np.random.default_rng(seed).integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    return words, torch.from_numpy(words.view(np.int32)).cuda()


def _xor(a):
    return int(np.bitwise_xor.reduce(a.astype(np.uint32))) if a.size else 0


@pytest.mark.parametrize("pattern", [0, 1, 2, 3])
@pytest.mark.parametrize("nbytes,grid", [(1 << 22, 64), (3 * (1 << 20) + 4096, 37)])
def test_stream_reads_cover_the_buffer_once(micro, pattern, nbytes, grid):
    words, buf = _buffer(nbytes, 1)
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    assert micro.moe_micro_hbm_read(vp(buf.data_ptr()), nbytes, vp(sink.data_ptr()), grid, pattern,
                                    vp(s.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert _xor(sink.cpu().numpy().view(np.uint32)) == _xor(words)


@pytest.mark.parametrize("group_kib,pad_kib", [(16, 0), (32, 0), (48, 0), (16, 1), (32, 1)])
@pytest.mark.parametrize("skew", [0, 1, 2])
@pytest.mark.parametrize("nt", [0, 1])
def test_gemm_group_reads_cover_each_group_once(micro, group_kib, pad_kib, skew, nt):
    gbytes, gstride = group_kib << 10, (group_kib + pad_kib) << 10
    region = 16 * gstride
    nreg = 11
    nbytes = nreg * region + 8192          # a tail past the last region that must not be read
    words, buf = _buffer(nbytes, 2)
    sink = torch.zeros(nreg * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    assert micro.moe_micro_hbm_read_groups(vp(buf.data_ptr()), nbytes, gbytes, gstride, skew,
                                           vp(sink.data_ptr()), nt, vp(s.cuda_stream)) == 0
    torch.cuda.synchronize()
    covered = np.zeros(nbytes // 4, dtype=bool)
    for r in range(nreg):
        for g in range(16):
            lo = (r * region + g * gstride) // 4
            covered[lo:lo + gbytes // 4] = True
    assert _xor(sink.cpu().numpy().view(np.uint32)) == _xor(words[covered])


def test_gemm_group_reads_refuse_bad_arguments(micro):
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    s = vp(torch.cuda.current_stream().cuda_stream)
    b, o = vp(buf.data_ptr()), vp(sink.data_ptr())
    assert micro.moe_micro_hbm_read_groups(b, 1 << 20, 6144, 6144, 0, o, 0, s) == 1      # not a multiple of 4 KiB
    assert micro.moe_micro_hbm_read_groups(b, 1 << 20, 2048, 2048, 0, o, 0, s) == 1      # below 4 KiB
    assert micro.moe_micro_hbm_read_groups(b, 1 << 20, 16 << 10, 8 << 10, 0, o, 0, s) == 1  # stride below the group
    assert micro.moe_micro_hbm_read_groups(b, 1 << 20, 16 << 10, 16 << 10, 3, o, 0, s) == 1  # unknown skew
    assert micro.moe_micro_hbm_read_groups(b, 1 << 17, 16 << 10, 16 << 10, 0, o, 0, s) == 1  # smaller than a region
