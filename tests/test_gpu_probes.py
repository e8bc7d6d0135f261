"""The two measurement probes bench.py --mfma-ceiling / --hbm-ceiling time,
run small on the GPU with results that have closed forms: all-ones bf16
operands give every accumulator element 16 per MFMA, and the XOR fold of
the read probe equals the XOR of every 32-bit word it read."""
import ctypes

import numpy as np
import pytest
import torch

from speculative_decoding_sd_amd import build as sdv_build
from parity import DEV

pytestmark = pytest.mark.gpu


def _probe_lib():
    P = ctypes.CDLL(sdv_build.PROBE_LIB_PATH)
    P.sdv_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    P.sdv_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    return P


def test_mfma_probe_all_ones():
    P = _probe_lib()
    blocks, iters = 3, 5
    ops = torch.ones(12 * 512 * 8, dtype=torch.bfloat16, device=DEV)
    sink = torch.full((blocks * 512,), -1.0, dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert P.sdv_probe_mfma_bf16(ops.data_ptr(), ops.numel() * 2, sink.data_ptr(), sink.numel(),
                                 blocks, iters, s) == 0
    torch.cuda.synchronize()
    # 8 accumulators x 16 registers per lane, each element 16 (k) per MFMA,
    # two k-steps per iteration.
    assert torch.all(sink == float(8 * 16 * 16 * 2 * iters))


def test_hbm_probe_xor_fold():
    P = _probe_lib()
    rng = np.random.default_rng(11)
    n_words = (1 << 16) + 8 * 256 * 3 + 5  # full tiles plus a ragged tail
    host = rng.integers(0, 2 ** 32, size=n_words * 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    for blocks in (1, 7, 64):
        sink = torch.zeros(blocks * 256, dtype=torch.int32, device=DEV)
        s = torch.cuda.current_stream().cuda_stream
        assert P.sdv_probe_hbm_read(src.data_ptr(), n_words * 16, sink.data_ptr(), sink.numel(),
                                    blocks, s) == 0
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), blocks
