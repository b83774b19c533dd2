"""ctypes view of libpa.so, the C ABI declared in include/pa.h.

The shared library is built in-tree next to this file.  Loading fails loudly
when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32, PA_BF16 = 0, 1
PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_ELAUNCH, PA_ESCRATCH = 0, -1, -2, -3, -4, -5

# every symbol include/pa.h declares, with its ctypes signature
_P = ctypes.c_void_p
_I = ctypes.c_int32
PA_HINT_UNSHARED = 1
PA_HEAD_MAJOR = 0x100   # pool layout flag OR-ed into the dtype argument
PA_WORKSPACE_HEADER = 4096
PA_NOALLOC_SCRATCH_BYTES = 32 << 20

SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_store_kv": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pa_copy_pages": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pa_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                 ctypes.c_float, _I, _P, ctypes.POINTER(ctypes.c_size_t), _P]),
    "pa_decode_sinks": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                       _I, _I, ctypes.c_float, _I, _P,
                                       ctypes.POINTER(ctypes.c_size_t), _P]),
    "pa_decode_hinted": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                        _I, _I, _I, ctypes.c_float, _I, _P,
                                        ctypes.POINTER(ctypes.c_size_t), _P]),
    "pa_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                  _I, _I, _I, ctypes.c_float, _I, _P,
                                  ctypes.POINTER(ctypes.c_size_t), _P]),
    "pa_prefill_hinted": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I,
                                         _I, _I, _I, _I, _I, ctypes.c_float, _I, _P,
                                         ctypes.POINTER(ctypes.c_size_t), _P]),
    "pa_update_tables": (ctypes.c_int, [_P, _I, _I, _P, _I, _I, _I, _P, _P, _P, _I, _I, _P]),
    "pa_reset_workspace": (ctypes.c_int, [_P, ctypes.c_size_t, _P]),
    "pa_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                         _I, _I, _I, ctypes.c_float, _I, _P]),
}

_lib = None


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def load() -> ctypes.CDLL:
    """The loaded library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(fn, status)
