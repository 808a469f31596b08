"""ctypes loader for libmga_gqa.so (the C ABI declared in include/mga_gqa.h).

The library is built in-tree by ``gqa_attention_split_amd.build``. There is no
fallback: if the shared object is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmga_gqa.so")

# Every symbol the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
_S = ctypes.c_size_t
_F = ctypes.c_float
SIGNATURES = {
    "mga_status_string": ([_I], ctypes.c_char_p),
    "mga_gqa_choose_splits": ([_I, _I, _I, _I], _I),
    "mga_gqa_effective_splits": ([_I, _I, _I, _I, _I], _I),
    "mga_gqa_workspace_bytes": ([_I, _I, _I, _I, _I], _S),
    "mga_gqa_plan": ([_I, _I, _I, _I, _I, _P, _P], _I),
    "mga_gqa_check_args": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S], _I),
    "mga_gqa_forward": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P], _I),
    "mga_gqa_partial": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P], _I),
    "mga_gqa_combine": ([_P, _I, _I, _I, _I, _I, _P, _S, _P], _I),
    "mga_gqa_forward_strided": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P, _S, _P], _I),
    "mga_gqa_check_args_strided": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P, _S], _I),
    "mga_gqa_forward_noalloc": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P], _I),
    "mga_gqa_qknorm_forward": ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _I, _P, _S, _P], _I),
    "mga_gqa_qknorm_workspace_bytes": ([_I, _I, _I, _I, _I], _S),
    "mga_gqa_qknorm_plan": ([_I, _I, _I, _I, _I, _P, _P], _I),
    "mga_gqa_qknorm_check_args": ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _I, _P, _S], _I),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gqa_attention_split_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib
