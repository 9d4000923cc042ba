"""ctypes view of libmoe.so (the C ABI declared in include/libmoe.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LIBMOE_PATH", os.path.join(PKG, "libmoe.so"))

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

# every symbol include/libmoe.h declares
EXPORTS = ("moe_router", "moe_gate", "moe_gate_record", "moe_stage_to_host", "moe_permute", "moe_grouped_ffn",
           "moe_grouped_ffn_traced", "moe_grouped_ffn_noalloc", "moe_grouped_ffn_combine",
           "moe_grouped_ffn_packed", "moe_grouped_ffn_fp8w",
           "moe_grouped_ffn_fp8w_packed", "moe_combine",
           "moe_stats", "moe_prob_signature", "moe_status_string")

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.POINTER(ctypes.c_size_t)

SIGNATURES = {
    "moe_router": [_p, _p, _i32, _i32, _i32, _i32, _p, _p],
    "moe_gate": [_p, _i32, _i32, _i32, _i32, _p, _p, _p],
    "moe_gate_record": [_p, _i32, _i32, _i32, _i32, _p, _p, _i32, _i32, _i32, _p, _p],
    "moe_stage_to_host": [_p, _p, ctypes.c_size_t, _p],
    "moe_permute": [_p, _i32, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p, _p, _p, _p, _p, _p, _sz, _p],
    "moe_grouped_ffn": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p, _sz, _p],
    "moe_grouped_ffn_traced": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p, _sz,
                               _p, _i32, _i32, _p],
    "moe_grouped_ffn_combine": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p, _i32,
                                _i32, _p, _p, _sz, _p],
    "moe_grouped_ffn_noalloc": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p],
    "moe_grouped_ffn_packed": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p],
    "moe_combine": [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p, _p],
    "moe_stats": [_p, _i32, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p],
    "moe_prob_signature": [_p, _i32, _i32, _i32, _p, _i32, _p, _p],
    "moe_grouped_ffn_fp8w": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                             _sz, _p],
    "moe_grouped_ffn_fp8w_packed": [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                             _sz, _p],
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so once.  Raises ImportError if it has not been built.

    torch must be imported first on a machine with a GPU so that the library binds to the
    same HIP runtime as torch's allocator and streams.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmoe.so not found at {path}: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
