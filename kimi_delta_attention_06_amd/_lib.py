"""ctypes loader for libkda.so (the HIP library built in-tree by build.py).

There is no fallback: if the library is missing or does not export the
expected symbols, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "kda.h")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_LAUNCH = 0, 1, 2, 3
KDA_DTYPE_F32, KDA_DTYPE_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 256 << 20  # KDA_NOALLOC_SCRATCH_BYTES

# Every function include/kda.h declares, with its ctypes signature.
_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "kda_chunk_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32,
                                     ctypes.c_int, _P, _P, _P]),
    "kda_chunk_fwd_checkpointed": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32,
                                                  _I32, ctypes.c_int, _P, _P, _I32, _P, _P]),
    "kda_chunk_fwd_split": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32,
                                           _I32, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P]),
    "kda_chunk_fwd_auto": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32,
                                          _I32, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P]),
    "kda_chunk_fwd_split_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32,
                                                   _I32, ctypes.c_int, _P, _P, _P]),
    "kda_chunk_fwd_split_workspace_size": (ctypes.c_int, [_I32, _I64, _I32, _I32, _I32, _I32, ctypes.c_int,
                                                          ctypes.POINTER(ctypes.c_size_t)]),
    "kda_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, ctypes.c_int,
                               _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "kda_bwd_workspace_size": (ctypes.c_int, [_I32, _I64, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "kda_bwd_recurrent": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, ctypes.c_int,
                                         _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "kda_bwd_recurrent_workspace_size": (ctypes.c_int, [_I32, _I64, _I32, _I32, _I32,
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "kda_recurrent_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                          ctypes.c_int, _P, _P]),
    "kda_recurrent_verify": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                            ctypes.c_int, _P, _P]),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_version": (ctypes.c_int32, []),
}

_lock = threading.Lock()
_lib = None


class KDALibraryError(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise KDALibraryError(
                    "libkda.so is not built (%s); run: python -m kimi_delta_attention_06_amd.build" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)  # AttributeError -> missing export
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load().kda_status_string(int(code)).decode()
