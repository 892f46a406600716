"""ctypes loader for libfa355.so (the C ABI declared in include/fa355.h).

The library is required: if it has not been built, every entry point raises
instead of falling back to any other implementation.  With FA355_DEBUG set in
the environment (to anything but "" or "0") the debug build,
libfa355_debug.so, is loaded instead: the same kernels, preceded by checks of
the callers' device arrays (see debug_flags in the package).
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
RELEASE_LIB_PATH = os.path.join(_HERE, "libfa355.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libfa355_debug.so")
LIB_PATH = (DEBUG_LIB_PATH if os.environ.get("FA355_DEBUG", "0") not in
            ("", "0") else RELEASE_LIB_PATH)

FA_F32, FA_BF16 = 0, 1
STATUS = {0: "FA_OK", -1: "FA_E_NULLPTR", -2: "FA_E_SHAPE",
          -3: "FA_E_UNSUPPORTED", -4: "FA_E_WORKSPACE", -5: "FA_E_HIP",
          -6: "FA_E_SCRATCH"}
FA_DECODE_SCRATCH_BYTES = 8 << 20

# Every function the header declares, with its ctypes signature.
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_U64, _U32 = ctypes.c_uint64, ctypes.c_uint32
SIGNATURES = {
    "fa_status_str": (ctypes.c_char_p, [_I]),
    "fa_last_hip_error": (_I, []),
    "fa_last_hip_error_str": (ctypes.c_char_p, []),
    "fa_debug_flags": (_I, [_P, _I]),
    "fa_fwd": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _F,
                    _P]),
    "fa_fwd_fp8": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                        _P, _P, _I, _F, _P]),
    "fa_bwd_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "fa_bwd_block_sparse_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _F,
                    _P, _P, _P, _P, _Z, _P]),
    "fa_fwd_dropout": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I,
                            _F, _F, _U64, _U32, _P]),
    "fa_bwd_dropout": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                            _I, _F, _F, _U64, _U32, _P, _P, _P, _P, _Z, _P]),
    "fa_fwd_block_sparse": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                 _I, _F, _P]),
    "fa_bwd_block_sparse": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _I, _F, _P, _P, _P, _P, _Z, _P]),
    "fa_fwd_varlen": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                           _P, _I, _F, _P]),
    "fa_bwd_varlen_workspace_bytes": (_Z, [_I, _I, _I]),
    "fa_bwd_varlen": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                           _P, _I, _F, _P, _P, _P, _P, _Z, _P]),
    "fa_prefill_paged": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I,
                              _I, _P, _I, _P, _I, _F, _P, _P, _P, _P]),
    "fa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P,
                             _I, _F, _P, _P, _Z, _P]),
    "fa_decode_paged_noalloc": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _I, _P,
                                     _I, _P, _I, _F, _P, _P]),
}


class LibraryMissing(RuntimeError):
    pass


class FaError(RuntimeError):
    def __init__(self, fn, status, detail=None):
        self.status = status
        msg = f"{fn} failed: {STATUS.get(status, status)}"
        super().__init__(msg if detail is None else f"{msg}: {detail}")


_lib = None


def load(path):
    """Open one build of the library and attach the declared signatures."""
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is not built: run "
            "`python -m exact_io_aware_15_amd.build` (needs ROCm hipcc)")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib():
    """The library every wrapper calls (loaded once, from LIB_PATH)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def check(fn, status):
    if status != 0:
        err = FaError(fn, status)
        if status == -5 and _lib is not None:   # FA_E_HIP: add HIP's reason
            why = _lib.fa_last_hip_error_str().decode()
            err = FaError(fn, status, f"{why} (hipError_t "
                                      f"{_lib.fa_last_hip_error()})")
        raise err
