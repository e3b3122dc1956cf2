"""ctypes view of libmla.so: symbol signatures exactly as include/mla.h declares."""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")
# The same library built with MLA_DEBUG_CHECKS: every decode entry point first
# checks its index arguments on the device, synchronises, and returns
# MLA_ERR_BAD_INPUT if they break the call's contract.
DEBUG_LIB_PATH = os.path.join(HERE, "libmla_debug.so")

STATUS = {
    0: "MLA_OK",
    1: "MLA_ERR_NULL_POINTER",
    2: "MLA_ERR_BAD_SHAPE",
    3: "MLA_ERR_BAD_DTYPE",
    4: "MLA_ERR_UNSUPPORTED",
    5: "MLA_ERR_WORKSPACE_TOO_SMALL",
    6: "MLA_ERR_HIP",
    7: "MLA_ERR_SCRATCH_TOO_SMALL",
    8: "MLA_ERR_BAD_INPUT",
}
# Bits of the word mla_check_inputs writes.
CHECK_BITS = {
    1: "MLA_CHECK_QO_INDPTR",
    2: "MLA_CHECK_KV_INDPTR",
    4: "MLA_CHECK_KV_INDEX",
    8: "MLA_CHECK_LAST_PAGE_LEN",
    16: "MLA_CHECK_DCP_LENGTHS",
}
DTYPE_FP8, DTYPE_BF16, DTYPE_FP32 = 0, 1, 2

_vp, _i32p, _f32p, _i64p = C.c_void_p, C.POINTER(C.c_int32), C.c_void_p, C.POINTER(C.c_int64)

_DECODE_ARGS = [
    _vp, C.c_int, _vp, C.c_int, C.c_int64, _vp, _vp, _vp, _vp, C.c_int64, _vp,
    C.c_int, C.c_int, C.c_int, C.c_int, C.c_float, _vp, _vp, C.c_int, _vp, _vp, C.c_size_t,
]

SIGNATURES = {
    "mla_decode": (C.c_int, _DECODE_ARGS + [_vp]),
    "mla_decode_ex": (C.c_int, _DECODE_ARGS + [C.c_int, _vp]),
    "mla_decode_noalloc": (C.c_int, _DECODE_ARGS[:20] + [_vp]),
    "mla_decode_noalloc_scratch_bytes": (C.c_size_t, []),
    "mla_decode_workspace_bytes": (C.c_size_t, [C.c_int] * 4),
    "mla_decode_workspace_bytes_ex": (C.c_size_t, [C.c_int] * 5),
    "mla_merge_partials": (C.c_int, [_vp, C.c_int, _vp, C.c_int, C.c_int, C.c_int, _vp, _vp, _vp]),
    "mla_status_string": (C.c_char_p, [C.c_int]),
    "mla_decode_cascade": (C.c_int, [
        _vp, C.c_int, _vp, C.c_int, C.c_int64, _vp, _vp, _vp, C.c_int64, _vp, _vp, C.c_int64,
        C.c_int, C.c_int, C.c_int, C.c_int, C.c_float, _vp, _vp, C.c_int, _vp, _vp, C.c_size_t,
        _vp]),
    "mla_decode_cascade_workspace_bytes": (C.c_size_t, [C.c_int] * 4),
    "mla_decode_paged": (C.c_int, _DECODE_ARGS[:11] + [C.c_int] + _DECODE_ARGS[11:] + [_vp]),
    "mla_decode_dcp": (C.c_int, _DECODE_ARGS[:20] + [_vp, C.c_int, C.c_int, C.c_int]
                       + _DECODE_ARGS[20:] + [_vp]),
    "mla_rope_quant_cache": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, C.c_int, C.c_int, _vp, C.c_int,
                                       C.c_int, C.c_int, _vp, C.c_int64, _vp, _vp, _vp, _vp]),
    "mla_latent_to_v": (C.c_int, [_vp, _vp, _vp, C.c_int, C.c_int, C.c_int, _vp]),
    "mla_decode_step_workspace_bytes": (C.c_size_t, [C.c_int] * 4),
    "mla_decode_step": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, C.c_int, C.c_int, _vp, _vp,
                                  C.c_int64, _vp, _vp, _vp, C.c_int64, C.c_int, C.c_int, C.c_int,
                                  C.c_int, C.c_int, C.c_float, _vp, _vp, _vp, _vp, _vp, C.c_int,
                                  _vp, _vp, C.c_size_t, _vp]),
    "mla_check_inputs": (C.c_int, [_vp, _vp, _vp, C.c_int64, _vp, C.c_int, C.c_int64, C.c_int,
                                   C.c_int, C.c_int, _vp, C.c_int, C.c_int, _vp, _vp]),
    "mla_plan_host": (C.c_int64, [_vp, _vp, _vp, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, _vp,
                                  C.c_int64]),
    "mla_plan_groups_host": (C.c_int64, [_vp, _vp, _vp, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                         C.c_int, _vp, C.c_int64]),
}

_lib = None
_debug_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def _load(path: str) -> C.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m mla_latent_attention_amd.build)"
        )
    handle = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib() -> C.CDLL:
    """Load libmla.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib() -> C.CDLL:
    """Load libmla_debug.so (the MLA_DEBUG_CHECKS build) once."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise MLAError(status, where)
