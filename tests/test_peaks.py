"""The benchmark's measurement kernels (libkda_peaks.so): the library loads and
exports its entry points (CPU), and on the GPU the streaming copy copies
exactly, the read stream and the matrix-core loop leave their sinks alone for
a key they never reach, and bad arguments are refused before any launch."""
import ctypes
import os

import pytest
import torch

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gated_delta_rule_38_amd", "libkda_peaks.so")


def load():
    if not os.path.exists(LIB):
        pytest.fail("libkda_peaks.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    vp, sz, i, u32, f = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32,
                         ctypes.c_float)
    lib.kda_peak_copy.argtypes = [vp, vp, sz, i, vp]
    lib.kda_peak_read.argtypes = [vp, sz, u32, vp, i, vp]
    lib.kda_peak_mfma.argtypes = [i, f, vp, i, vp]
    return lib


def test_exports():
    lib = load()
    for name in ("kda_peak_copy", "kda_peak_read", "kda_peak_mfma", "kda_peak_mfma_chains"):
        assert hasattr(lib, name)
    assert lib.kda_peak_mfma_chains() == 4


def test_rejects_bad_arguments_without_launching():
    lib = load()
    EINVAL = 1  # hipErrorInvalidValue
    assert lib.kda_peak_copy(16, 32, 17, 8, None) == EINVAL      # size not a multiple of 16
    assert lib.kda_peak_copy(8, 32, 32, 8, None) == EINVAL       # misaligned source
    assert lib.kda_peak_copy(16, 32, 32, 0, None) == EINVAL      # no workgroups
    assert lib.kda_peak_read(16, 32, 0, None, 8, None) == EINVAL  # no sink
    assert lib.kda_peak_mfma(0, 1.0, 64, 8, None) == EINVAL       # no iterations


@pytest.mark.gpu
def test_copy_exact_and_sinks_untouched():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = load()
    dev = torch.device("cuda:0")
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    n = (1 << 20) + 48  # bytes: a tail that no thread's full stride covers
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev, generator=g)
    dst = torch.zeros_like(src)
    blocks = 64
    assert lib.kda_peak_copy(src.data_ptr(), dst.data_ptr(), n, blocks, st) == 0
    sink = torch.full((blocks * 256,), 7.0, dtype=torch.float32, device=dev)
    ones = torch.ones(n // 4, dtype=torch.float32, device=dev)  # every 16-byte word XORs to 0
    assert lib.kda_peak_read(ones.data_ptr(), n, 0x9E3779B9, sink.data_ptr(), blocks, st) == 0
    assert lib.kda_peak_mfma(100, 12345.678, sink.data_ptr(), blocks, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert torch.all(sink == 7.0)
