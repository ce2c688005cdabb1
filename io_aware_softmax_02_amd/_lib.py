"""ctypes loader for ``libfa_mi355x.so`` and the prototypes of include/fa.h.

Importing this module raises if the library has not been built: there is no
fallback path of any kind.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa_mi355x.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_f = ctypes.c_float
_sz = ctypes.c_size_t
_st = ctypes.c_int

# name -> (restype, argtypes), in the order of include/fa.h
PROTOTYPES = {
    "fa_status_str": (ctypes.c_char_p, [_st]),
    "fa_fwd": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p]),
    "fa_fwd_split_max": (_i64, [_i64, _i64, _i64, _i64]),
    "fa_fwd_split": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _i64, _p]),
    "fa_merge": (_st, [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _p]),
    "fa_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fa_bwd": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                     _i64, _i64, _i64, _i64, _f, _p]),
    "fa_bwd_noalloc": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _p,
                             _i64, _i64, _i64, _i64, _f, _p]),
    "fa_bwd_preprocess": (_st, [_p, _p, _p, _i64, _i64, _i64, _i64, _p]),
    "fa_bwd_dkdv": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p]),
    "fa_bwd_dq": (_st, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p]),
    "fa_f32_key_block": (_i64, [_i64, _i64]),
    "fa_fwd_f32": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p]),
    "fa_bwd_f32_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fa_bwd_f32": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                         _i64, _i64, _i64, _i64, _f, _p]),
}


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python io_aware_softmax_02_amd/build.py` "
            "(the attention ops have no other implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = load()

# Status codes of include/fa.h
FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_UNSUPPORTED = 3
FA_ERR_ALIGN = 4
FA_ERR_WORKSPACE = 5
FA_ERR_SCALE = 6
FA_ERR_ALIAS = 7
FA_ERR_HIP = 8
FA_ERR_SCRATCH = 9
FA_BWD_NOALLOC_MAX_ROWS = 1 << 22


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def status_str(status: int) -> str:
    return LIB.fa_status_str(int(status)).decode()
