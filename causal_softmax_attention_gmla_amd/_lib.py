"""ctypes loader for libgmla.so (the HIP kernels and their C ABI, include/gmla.h).

The library is the only compute path: if it is missing or cannot be loaded, every
call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgmla.so")

GMLA_F32 = 0
GMLA_BF16 = 1

_STATUS = {0: "GMLA_OK", -1: "GMLA_ERR_INVALID_ARG", -2: "GMLA_ERR_UNSUPPORTED",
           -3: "GMLA_ERR_WORKSPACE", -4: "GMLA_ERR_HIP", -5: "GMLA_ERR_TOO_LARGE"}

# every symbol gmla.h declares, with its ctypes signature
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_i64p = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "gmla_status_string": (ctypes.c_char_p, [_i]),
    "gmla_version": (_i, []),
    "gmla_attend_prefill": (_i, [_i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _i64p, _vp, _vp, _vp]),
    "gmla_attend_chunk": (_i, [_i, _i, _i, _i, _i, _i, _f, _i, _vp, _i64p, _vp, _vp, _i64p, _vp,
                               _vp, _vp]),
    "gmla_prefill_latent_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "gmla_attend_prefill_latent": (_i, [_i, _i, _i, _i, _i, _i, _f, _i, _vp, _i64p, _vp, _vp, _vp,
                                        _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "gmla_attend_varlen": (_i, [_i, _i, _i, _i, _f, _i, _vp, _i64p, _vp, _i, _vp, _vp, _i64p, _vp,
                                _i, _vp, _vp, _vp]),
    "gmla_attend_decode_varlen": (_i, [_i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _i64p, _vp, _vp, _vp,
                                       _vp, ctypes.c_size_t, _i, _vp]),
    "gmla_decode_num_splits": (_i, [_i, _i, _i, _i]),
    "gmla_decode_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "gmla_attend_decode": (_i, [_i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _i64p, _vp, _vp, _vp,
                                ctypes.c_size_t, _i, _vp]),
    "gmla_decode_latent_num_splits": (_i, [_i, _i, _i, _i]),
    "gmla_decode_latent_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "gmla_attend_decode_latent": (_i, [_i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i64p, _vp, _vp, _vp,
                                       _vp, _vp, ctypes.c_size_t, _i, _vp]),
    "gmla_attend_decode_latent_varlen": (_i, [_i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i64p, _vp, _vp,
                                              _vp, _vp, _vp, _vp, ctypes.c_size_t, _i, _vp]),
    "gmla_decode_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "gmla_attend_decode_noalloc": (_i, [_i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _i64p, _vp, _vp, _i,
                                        _vp]),
    "gmla_latent_expand": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gmla_gate_out": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "gmla_gate_out_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "gmla_gate_out_ws": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "gmla_linear": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "gmla_linear_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "gmla_linear_ws": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
}

_lock = threading.Lock()
_lib: ctypes.CDLL | None = None


class GmlaError(RuntimeError):
    """A libgmla call returned a non-zero status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgmla.so once (raises if it was not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m causal_softmax_attention_gmla_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status != 0:
        raise GmlaError(status, what)
