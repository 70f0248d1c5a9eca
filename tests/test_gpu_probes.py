"""The bandwidth probes that set the measured peaks in bench.py (libkda_peaks.so) do what they
claim: the read stream sums every element it is given, the copy copies, and the in-place update
writes a x + b, on sizes with ragged tails.  Plus a host-only check that the library exports
its entry points."""
import ctypes

import pytest
import torch

from chunked_gated_delta_13_amd import build as kbuild

SYMBOLS = ("kda_peak_read_sink_floats", "kda_peak_read", "kda_peak_copy", "kda_peak_rmw")
RMW_BLOCK_FLOATS = 4096 * 4   # one 64 KiB block


def _lib():
    lib = ctypes.CDLL(kbuild.PEAKS_LIB)
    lib.kda_peak_read_sink_floats.restype = ctypes.c_size_t
    lib.kda_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.kda_peak_rmw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_void_p]
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_probe_library_exports():
    lib = ctypes.CDLL(kbuild.PEAKS_LIB)
    for name in SYMBOLS:
        assert hasattr(lib, name), name


# float counts: below one block, exact blocks, ragged tails, more blocks than 8 XCD ranges divide
SIZES = [4, 1000, RMW_BLOCK_FLOATS, 3 * RMW_BLOCK_FLOATS + 20, 37 * RMW_BLOCK_FLOATS - 4, 1 << 22]


@pytest.mark.gpu
@pytest.mark.parametrize("n", SIZES)
def test_probes_compute_what_they_claim(n):
    print(f"probes n={n}", flush=True)
    lib = _lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(n)
    x = torch.rand(n, generator=gen, device="cuda", dtype=torch.float32)

    sink = torch.full((lib.kda_peak_read_sink_floats(),), float("nan"), device="cuda")
    assert lib.kda_peak_read(_p(x), 4 * n, _p(sink), sp) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    ref = x.double().sum().item()
    assert abs(sink.double().sum().item() - ref) <= 1e-5 * ref

    dst = torch.full_like(x, float("nan"))
    assert lib.kda_peak_copy(_p(dst), _p(x), 4 * n, sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, x)

    y = x.clone()
    assert lib.kda_peak_rmw(_p(y), 4 * n, 2.0, 0.5, sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, x * 2.0 + 0.5)


@pytest.mark.gpu
def test_probes_reject_bad_arguments():
    lib = _lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    x = torch.zeros(64, device="cuda")
    sink = torch.zeros(lib.kda_peak_read_sink_floats(), device="cuda")
    assert lib.kda_peak_read(_p(x), 6, _p(sink), sp) == 1            # not a multiple of 16
    assert lib.kda_peak_copy(_p(x), _p(x[4:]), 64, sp) == 1           # overlapping
    assert lib.kda_peak_rmw(ctypes.c_void_p(x.data_ptr() + 4), 64, 1.0, 0.0, sp) == 1   # misaligned
    assert lib.kda_peak_rmw(_p(x), 0, 1.0, 0.0, sp) == 0              # nothing to do
