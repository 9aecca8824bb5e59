"""The streaming-read kernel of the achievable-HBM measurement reads every
16-byte word exactly once: the XOR of its per-workgroup results equals the
XOR of all 32-bit words of the buffer (numpy), for grids that leave ragged
tails."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "quantized_kv_flashattention_amd", "libqkvfa_bench.so")


@pytest.mark.parametrize("n_words,grid", [(4, 1), (4 * 1000, 3), (4 * 262147, 64), (4 * (1 << 20), 1024)])
def test_stream_read_reads_every_word_once(n_words, grid):
    lib = ctypes.CDLL(LIB)
    lib.qkvb_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    rng = np.random.default_rng(n_words + grid)
    host = rng.integers(0, 2 ** 32, size=n_words, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(grid, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.qkvb_stream_read(src.data_ptr(), n_words * 4, out.data_ptr(), grid, st) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
