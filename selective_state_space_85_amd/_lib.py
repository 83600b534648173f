"""ctypes view of libssscan.so (the C ABI declared in include/ss_scan.h).

Only loads what ``build.py`` produced in this directory; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssscan.so")

SS_OK, SS_ERR_INVALID_ARG, SS_ERR_UNSUPPORTED, SS_ERR_WORKSPACE, SS_ERR_HIP = range(5)
SS_F32, SS_BF16 = 0, 1

# Every function the header declares.
EXPORTS = ("ss_scan_plan", "ss_scan_plan_ex", "ss_scan_workspace_bytes", "ss_scan_workspace_bytes_ex", "ss_scan_fwd", "ss_scan_fwd_ex",
           "ss_scan_fwd_noalloc", "ss_scan_ckpt_bytes",
           "ss_scan_fwd_ckpt", "ss_step", "ss_step_ex", "ss_scan_bwd_workspace_bytes", "ss_scan_bwd",
           "ss_scan_bwd_ckpt_workspace_bytes", "ss_scan_bwd_ckpt", "ss_conv1d_silu", "ss_ssd_fwd", "ss_ssd_fwd_ex", "ss_ssd_workspace_bytes",
           "ss_status_string", "ss_last_hip_error")
SS_DELTA_SOFTPLUS, SS_B_ZOH = 1, 2  # ss_option bits
SS_NOALLOC_MAX_WORKSPACE_BYTES = 32 << 20  # ss_scan_fwd_noalloc's per-GPU array

_lib = None


class SSError(RuntimeError):
    """A non-SS_OK status from the library."""

    def __init__(self, fn: str, status: int, hip_error: int = 0):
        msg = "%s: %s" % (fn, status_string(status))
        if status == SS_ERR_HIP:
            msg += " (hipError_t %d)" % hip_error
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


def load() -> ctypes.CDLL:
    """Load libssscan.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libssscan.so is not built (%s); run "
                           "`python -m selective_state_space_85_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.ss_scan_plan.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.ss_scan_plan.restype = ctypes.c_int
    lib.ss_scan_plan_ex.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.ss_scan_plan_ex.restype = ctypes.c_int
    lib.ss_scan_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.ss_scan_workspace_bytes.restype = sz
    lib.ss_scan_workspace_bytes_ex.argtypes = [i64, i64, i64, i64, i64]
    lib.ss_scan_workspace_bytes_ex.restype = sz
    lib.ss_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                i64, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_scan_fwd.restype = ctypes.c_int
    lib.ss_scan_fwd_noalloc.argtypes = [vp] * 10 + [i64, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ss_scan_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp, vp, sz,
                                   i64, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_scan_fwd_ex.restype = ctypes.c_int
    lib.ss_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_step.restype = ctypes.c_int
    lib.ss_step_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, i64, i64, i64,
                               ctypes.c_int, vp]
    lib.ss_step_ex.restype = ctypes.c_int
    lib.ss_scan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.ss_scan_bwd_workspace_bytes.restype = sz
    lib.ss_scan_bwd.argtypes = [vp] * 9 + [ctypes.c_uint32] + [vp] * 12 + [sz, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_scan_bwd.restype = ctypes.c_int
    lib.ss_scan_ckpt_bytes.argtypes = [i64, i64, i64, i64]
    lib.ss_scan_ckpt_bytes.restype = sz
    lib.ss_scan_fwd_ckpt.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp, vp, vp, sz,
                                     i64, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_scan_fwd_ckpt.restype = ctypes.c_int
    lib.ss_scan_bwd_ckpt_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.ss_scan_bwd_ckpt_workspace_bytes.restype = sz
    lib.ss_scan_bwd_ckpt.argtypes = [vp] * 9 + [ctypes.c_uint32] + [vp] * 13 + [sz, i64, i64, i64, i64, ctypes.c_int,
                                                                               vp]
    lib.ss_scan_bwd_ckpt.restype = ctypes.c_int
    lib.ss_conv1d_silu.argtypes = [vp, i64, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.ss_conv1d_silu.restype = ctypes.c_int
    lib.ss_ssd_fwd.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_int, vp]
    lib.ss_ssd_fwd.restype = ctypes.c_int
    lib.ss_ssd_fwd_ex.argtypes = [vp] * 10 + [ctypes.c_size_t] + [i64] * 5 + [ctypes.c_int, vp]
    lib.ss_ssd_fwd_ex.restype = ctypes.c_int
    lib.ss_ssd_workspace_bytes.argtypes = [i64] * 5
    lib.ss_ssd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_status_string.argtypes = [ctypes.c_int]
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_last_hip_error.argtypes = []
    lib.ss_last_hip_error.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().ss_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != SS_OK:
        raise SSError(fn, status, load().ss_last_hip_error() if status == SS_ERR_HIP else 0)
