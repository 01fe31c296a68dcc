"""ctypes binding of libsqa.so (include/sqa.h). Argument marshalling only:
every step of the computation runs in the library's HIP kernels."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsqa.so")

SQA_OK, SQA_ERR_INVALID_ARG, SQA_ERR_UNSUPPORTED, SQA_ERR_HIP, SQA_ERR_OUT_OF_MEMORY = range(5)
SQA_DTYPE_FP32, SQA_DTYPE_BF16 = 0, 1

# Every function the header declares, with its ctypes signature.
_i64, _vp, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "sqa_forward": (_int, [_vp] * 6 + [_i64] * 7 + [_int, _int, _vp]),
    "sqa_forward_noalloc": (_int, [_vp] * 6 + [_i64] * 7 + [_int, _int, _vp]),
    "sqa_forward_varlen": (_int, [_vp] * 7 + [_i64] * 7 + [_int, _int, _vp]),
    "sqa_prefill": (_int, [_vp] * 8 + [_i64] * 8 + [_int, _vp]),
    "sqa_decode_step": (_int, [_vp] * 9 + [_i64] * 7 + [_int, _vp]),
    "sqa_training_saved_bytes": (ctypes.c_size_t, [_i64] * 5 + [_int]),
    "sqa_forward_train": (_int, [_vp] * 7 + [ctypes.c_size_t] + [_i64] * 7 + [_int, _int, _vp]),
    "sqa_backward": (_int, [_vp] * 7 + [ctypes.c_size_t] + [_vp] * 5 + [_i64] * 7
                     + [_int, _int, _vp]),
    "sqa_padded_length": (_i64, [_i64]),
    "sqa_qkv_projection": (_int, [_vp] * 7 + [_i64] * 7 + [_int, _vp]),
    "sqa_attention": (_int, [_vp] * 4 + [_i64] * 5 + [_int, _int, _vp]),
    "sqa_output_projection": (_int, [_vp] * 3 + [_i64] * 3 + [_int, _vp]),
    "sqa_status_string": (ctypes.c_char_p, [_int]),
    "sqa_last_error_message": (ctypes.c_char_p, []),
}


class SQAError(RuntimeError):
    """A HIP failure or workspace allocation failure reported by libsqa."""


_lib = None


def load() -> ctypes.CDLL:
    """Load libsqa.so once. Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    """Map a non-OK sqa_status to a Python exception carrying the library's detail."""
    if status == SQA_OK:
        return
    lib = load()
    msg = f"{lib.sqa_status_string(status).decode()}: {lib.sqa_last_error_message().decode()}"
    if status == SQA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == SQA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise SQAError(msg)
