"""ctypes loader for liblapattn.so (the C ABI declared in include/lapattn.h).

Loading fails loudly: there is no fallback implementation of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblapattn.so")

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_M_TOO_LARGE = -3
ERR_PARAM = -4
ERR_DTYPE = -5
ERR_ALIAS = -6
ERR_WORKSPACE = -7
ERR_HIP = -8
ERR_ALIGN = -9
ERR_SCRATCH = -10
NOALLOC_SCRATCH_BYTES = 128 << 20

KERNEL_LAPLACIAN = 0
KERNEL_GAUSSIAN = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
FLAG_SERIAL = 1
FLAG_TICKETS = 2
SOLVER_NEWTON_SCHULZ = 0
SOLVER_CG = 1

# Names of every entry point declared in include/lapattn.h.
EXPORTS = ("lapattn_version", "lapattn_strerror", "lapattn_check",
           "lapattn_workspace_bytes", "lapattn_status_offset", "lapattn_init",
           "lapattn_forward", "lapattn_forward_noalloc",
           "lapattn_backward_workspace_bytes", "lapattn_backward", "lapattn_landmark_solve",
           "lapattn_block_workspace_bytes", "lapattn_block_forward",
           "lapattn_forward_normalized",
           "lapattn_forward_stages", "lapattn_set_stage_events", "lapattn_launches")

STAGES = ("pool", "main", "maps", "out", "bwd_part", "bwd_head", "bwd_grad", "bwd_dk")


class Desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("pool_h", ctypes.c_int32),
        ("pool_w", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class LapattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"lapattn error {status}: {message}")
        self.status = status


class LapattnTimeout(RuntimeError):
    """A forward call's in-launch waits ran out of time: its output is invalid."""

    def __init__(self, count: int):
        super().__init__(f"lapattn: {count} in-launch wait(s) timed out; the output is invalid")
        self.count = count


_lib = None
_lock = threading.Lock()


def _declare(lib):
    vp, fp, i32, f32, sz = (ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                            ctypes.c_int32, ctypes.c_float, ctypes.c_size_t)
    dp = ctypes.POINTER(Desc)
    lib.lapattn_version.argtypes = []
    lib.lapattn_version.restype = ctypes.c_int
    lib.lapattn_strerror.argtypes = [ctypes.c_int]
    lib.lapattn_strerror.restype = ctypes.c_char_p
    lib.lapattn_check.argtypes = [dp, f32, f32, i32]
    lib.lapattn_check.restype = ctypes.c_int
    lib.lapattn_workspace_bytes.argtypes = [dp]
    lib.lapattn_workspace_bytes.restype = sz
    lib.lapattn_status_offset.argtypes = [dp]
    lib.lapattn_status_offset.restype = sz
    lib.lapattn_init.argtypes = []
    lib.lapattn_init.restype = ctypes.c_int
    lib.lapattn_forward.argtypes = [dp, vp, vp, vp, f32, f32, i32, vp, vp, sz, vp]
    lib.lapattn_forward.restype = ctypes.c_int
    lib.lapattn_backward_workspace_bytes.argtypes = [dp, i32]
    lib.lapattn_backward_workspace_bytes.restype = sz
    lib.lapattn_backward.argtypes = [dp, vp, vp, vp, vp, f32, f32, i32, vp, vp, vp, vp, sz, vp]
    lib.lapattn_backward.restype = ctypes.c_int
    lib.lapattn_landmark_solve.argtypes = [dp, vp, vp, f32, f32, i32, i32, vp, vp]
    lib.lapattn_landmark_solve.restype = ctypes.c_int
    lib.lapattn_block_workspace_bytes.argtypes = [dp, i32]
    lib.lapattn_block_workspace_bytes.restype = sz
    lib.lapattn_block_forward.argtypes = [dp, i32, vp, vp, vp, vp, vp, f32, f32, i32, vp, vp, sz, vp]
    lib.lapattn_block_forward.restype = ctypes.c_int
    lib.lapattn_forward_normalized.argtypes = [dp, vp, vp, vp, f32, f32, i32, f32, vp, vp, sz, vp]
    lib.lapattn_forward_normalized.restype = ctypes.c_int
    lib.lapattn_forward_noalloc.argtypes = [dp, vp, vp, vp, f32, f32, i32, vp, vp, vp]
    lib.lapattn_forward_noalloc.restype = ctypes.c_int
    lib.lapattn_forward_stages.argtypes = [dp, vp, vp, vp, f32, f32, i32, vp, vp, sz, vp,
                                           vp, vp, vp, vp, vp, vp]
    lib.lapattn_forward_stages.restype = ctypes.c_int
    lib.lapattn_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.lapattn_set_stage_events.restype = ctypes.c_int
    lib.lapattn_launches.argtypes = [dp, ctypes.c_int]
    lib.lapattn_launches.restype = ctypes.c_int
    return lib


def lib():
    """The loaded library; raises if liblapattn.so has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m nystr_linear_attention_amd.build` (hipcc, gfx950)")
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def strerror(status: int) -> str:
    return lib().lapattn_strerror(status).decode()


def check(status: int) -> None:
    if status != OK:
        raise LapattnError(status, strerror(status))
