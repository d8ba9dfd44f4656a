"""ctypes loader for libfa.so and the C-ABI symbol table.

The library is loaded from this package directory. There is no fallback: if the
shared library is missing or does not load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

c_void_p, c_int, c_float, c_size_t = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fa.h
SIGNATURES = {
    "fa_status_string": (ctypes.c_char_p, [c_int]),
    "fa_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                       c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p]),
    "fa_fwd_f32out": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p]),
    "fa_decode_default_splits": (c_int, [c_int, c_int, c_int, c_int]),
    "fa_decode_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "fa_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                          c_int, c_int, c_int, c_int, c_int, c_float,
                          c_int, c_void_p, c_size_t, c_void_p]),
    "fa_decode_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_void_p]),
    "fa_decode_partials": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_void_p]),
    "fa_decode_combine": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int, c_int, c_int, c_int, c_void_p]),
    "fa_decode_paged": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float,
                                c_int, c_void_p, c_size_t, c_void_p]),
    "fa_bwd_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "fa_bpt_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "fa_bpt_layer": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_void_p, c_size_t,
                             c_void_p]),
    "fa_fwd_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                           c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p]),
    "fa_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                       c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, c_size_t, c_void_p]),
}

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP = range(7)

_lib = None


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise ImportError with the reason if it cannot be loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run io_aware_exact_21_amd.build.build() "
                          "(or __graft_entry__.build()) first")
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise ImportError(f"cannot load {LIB_PATH}: {e}") from e
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class FaError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().fa_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)
