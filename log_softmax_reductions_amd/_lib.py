"""ctypes loader for liblse.so and the raw C-ABI signatures of include/lse.h."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblse.so")

# Every symbol include/lse.h and include/lse_testing.h declare, with (restype,
# argtypes).
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
SIGNATURES = {
    "lse_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lse_last_error": (ctypes.c_char_p, []),
    "lse_abi_version": (ctypes.c_int, []),
    "lse_reduce_axis0": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "lse_reduce_axis": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "log_softmax_axis": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "lse_reduce_axis_strided": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                               _vp]),
    "log_softmax_axis_strided": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                                _i64, _vp]),
    "lse_axis_workspace_bytes": (_sz, [_i64, _i64, _i64, ctypes.c_int]),
    "lse_reduce_axis0_ws": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    "lse_reduce_axis_strided_ws": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                                  _vp, _sz, _vp]),
    "log_softmax_axis_strided_ws": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                                   _i64, _vp, _sz, _vp]),
    "log_softmax_rows_strided": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    "softmax_rows_strided": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    "log_softmax_rows_workspace_bytes": (_sz, [_i64, _i64]),
    "softmax_rows": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    "log_softmax_rows": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    "log_softmax_rows_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "lse_testing_set_spin_limit": (None, [ctypes.c_uint32]),
    "lse_testing_set_chain_path": (ctypes.c_int, [ctypes.c_int]),
    "lse_testing_set_rows_reread": (None, [ctypes.c_int]),
    "log_softmax_rows_plan": (ctypes.c_int, [_i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "lse_rows_num_chunks": (_i64, [_i64, _i64]),
    "lse_rows_partial": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "lse_rows_merge": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "fused_conv_gn_act_lse_workspace_bytes": (_sz, [_i64] * 7),
    "fused_conv_gn_act_lse": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                             _i64, _i64, _i64, ctypes.c_float, _vp, _vp, _sz,
                                             _vp]),
}

_lib = None


class LseError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed: {status_name(status)}: {detail}")


def load() -> ctypes.CDLL:
    """Load the in-tree liblse.so (never a fallback: raises if it is missing)."""
    global _lib
    if _lib is None:
        # Load the HIP runtime torch ships first, so the library binds to the
        # same runtime (and stream objects) as torch's allocator.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run log_softmax_reductions_amd/build.py "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_name(status: int) -> str:
    return load().lse_status_string(int(status)).decode()


def check(status: int, func: str) -> None:
    if status != 0:
        raise LseError(status, func, load().lse_last_error().decode())
