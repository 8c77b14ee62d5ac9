"""ctypes loader for libkda.so (the C ABI declared in include/kda.h).

The library is built in-tree by ``gated_delta_rule_64_amd.build``.  There is
no fallback: if the shared object is missing or fails to load, every entry
point raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_HIP = 4
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20  # mirrors kda.h
KDA_F32 = 0
KDA_BF16 = 1

# name -> (restype, argtypes); mirrors include/kda.h
_i32, _i64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
PROTOTYPES = {
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_last_error_detail": (ctypes.c_char_p, []),
    "kda_abi_version": (ctypes.c_int, []),
    "kda_preprocess": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32] + [_vp] * 8 + [_vp] + [_vp] * 5 + [_vp]),
    "kda_prefill_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32]),
    "kda_prefill_chunked": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32, _i32] + [_vp] * 6 +
                            [_vp, _vp, _vp, _vp, _sz, _vp]),
    "kda_decode_step": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 6 + [_vp, _vp, _vp]),
    "kda_prefill_layer": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32] + [_vp] * 8 +
                          [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kda_prefill_layer_noalloc": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32] + [_vp] * 8 +
                                  [_vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_decode_layer": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32] + [_vp] * 8 + [_vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "kda_spec_draft_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "kda_backward_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "kda_prefill_backward": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32, _i32] + [_vp] * 7 +
                             [_vp, _vp] + [_vp] * 7 + [_vp, _sz, _vp]),
    "kda_prefill_chunked_snap": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32, _i32] + [_vp] * 6 +
                                 [_vp, _vp, _vp, _vp, _sz, _i32, _vp, _i64, _vp, _vp]),
    "kda_prefill_layer_snap": (ctypes.c_int, [_i64, _i32, _i32, _i32, _vp, _i32, _i32] + [_vp] * 8 +
                               [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i32, _vp, _i64, _vp, _vp]),
    "kda_spec_verify": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 8 +
                        [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]),
}


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


PROTOTYPES["kda_profile_enable"] = (ctypes.c_int, [ctypes.c_int])
PROTOTYPES["kda_profile_collect"] = (ctypes.c_int, [ctypes.POINTER(KernelTime), ctypes.c_int])
PROTOTYPES["kda_probe_peak"] = (ctypes.c_int, [_i32, _i32, _i32, _vp, _i64, _vp, _vp])


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{status_string(status)}: {detail}")


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkda is not built ({LIB_PATH} missing); run __graft_entry__.build() "
                               "or python -m gated_delta_rule_64_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().kda_status_string(status).decode()


def check(status: int) -> None:
    if status != KDA_OK:
        raise KdaError(status, lib().kda_last_error_detail().decode())


def profile_enable(on: bool) -> None:
    """Per-kernel HIP-event timing of later calls on this thread (see kda.h)."""
    lib().kda_profile_enable(1 if on else 0)


def profile_collect() -> dict:
    """{kernel name: (launches, total ms)} since the last collect."""
    buf = (KernelTime * 64)()
    n = lib().kda_profile_collect(buf, 64)
    if n < 0:
        raise KdaError(-n, "event timing failed")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}
