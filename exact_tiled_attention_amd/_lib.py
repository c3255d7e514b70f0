"""ctypes view of libattn.so: symbol prototypes only (no computation here)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_F16, ATTN_BF16, ATTN_F32, ATTN_FP8_E4M3 = 0, 1, 2, 3
STATUS = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_GQA",
    -4: "ATTN_ERR_HEADDIM", -5: "ATTN_ERR_DTYPE", -6: "ATTN_ERR_WORKSPACE",
    -7: "ATTN_ERR_HIP", -8: "ATTN_ERR_ARG",
}

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
_U64 = ctypes.c_ulonglong
_U32 = ctypes.c_uint
_LL = ctypes.c_longlong

PROTOTYPES = {
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_fwd_exp_emulated": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "attn_exp2_soft": (_I, [_P, _P, _LL, _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_fp8_kv_tile": (_I, []),
    "attn_bwd_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P, _S, _P]),
    "attn_bwd_atomic": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P, _S, _P]),
    "attn_fp8_quantize": (_I, [_P, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P]),
    "attn_fwd_dropout": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _F, _U64, _U32, _I, _P]),
    "attn_bwd_dropout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _F, _U64, _U32,
                              _I, _I, _I, _I, _P, _S, _P]),
    "attn_bwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S,
                          _P]),
    "attn_bwd_deterministic_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_bwd_deterministic": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I,
                                    _P, _S, _P]),
    "attn_decode_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "attn_decode_pick_chunk": (_I, [_I, _I, _I]),
    "attn_decode_splitkv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]),
    "attn_decode_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]),
    "attn_tile_plan": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libattn.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -m exact_tiled_attention_amd.build`")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(cdll, name)
            fn.restype = res
            fn.argtypes = args
        _lib = cdll
    return _lib


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: "
                         f"{lib().attn_status_string(status).decode()}")


def check(fn: str, status: int) -> None:
    if status != 0:
        raise AttnError(fn, status)
