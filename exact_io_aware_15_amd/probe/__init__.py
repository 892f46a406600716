"""ctypes binding of libfa355_probe.so (include/fa355_probe.h): the
attainable bf16 matrix-core rate with the engine clock under that load, and
the streaming read rate of device memory.  Measurement context for the
attention kernels, not part of their path."""

import ctypes
import os

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__))), "libfa355_probe.so")

_D = ctypes.POINTER(ctypes.c_double)
SIGNATURES = {
    "fa_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _D, _D,
                                          _D]),
    "fa_probe_read_bw": (ctypes.c_int, [ctypes.c_size_t, ctypes.c_int, _D]),
}
_handle = None


def lib():
    global _handle
    if _handle is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built: run "
                               "`python -m exact_io_aware_15_amd.build`")
        h = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _handle = h
    return _handle


def mfma_bf16(iters=40000, waves_per_simd=2):
    """(TFLOP/s, engine clock GHz, seconds) of a pure bf16 MFMA loop on
    every SIMD of the current device."""
    t, c, s = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    st = lib().fa_probe_mfma_bf16(iters, waves_per_simd, ctypes.byref(t),
                                  ctypes.byref(c), ctypes.byref(s))
    if st != 0:
        raise RuntimeError(f"fa_probe_mfma_bf16 failed: {st}")
    return t.value, c.value, s.value


def read_bw(nbytes=1 << 30, reps=5):
    """Streaming read rate of device memory in GB/s."""
    g = ctypes.c_double()
    st = lib().fa_probe_read_bw(nbytes, reps, ctypes.byref(g))
    if st != 0:
        raise RuntimeError(f"fa_probe_read_bw failed: {st}")
    return g.value
