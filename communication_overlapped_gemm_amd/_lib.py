"""ctypes declarations of the C ABI in include/ocg.h (argument marshalling only).

The library is loaded after torch so that it binds to the same HIP runtime
instance as torch (both export the soname libamdhip64.so.7); stream handles
and device pointers from torch are then valid in every call. Loading fails
loudly if the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (loads the HIP runtime first, see above)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libocg.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_SHAPE = -2
ERR_WORKSPACE_TOO_SMALL = -3
ERR_HIP = -4
ERR_TIMEOUT = -5
ERR_NO_DEVICE = -6

OP_AG_GEMM, OP_GEMM_RS, OP_AG_GROUPED_GEMM, OP_MOE_COMBINE_RS, OP_AG_ATTENTION = 0, 1, 2, 3, 4
MODE_FUSED, MODE_GEMM_ONLY, MODE_COPY_ONLY = 0, 1, 2
TRANSFER_AUTO, TRANSFER_INLINE, TRANSFER_SIDE = -1, 0, 1
TILE_AUTO, TILE_256x224, TILE_128x224, TILE_128x256, TILE_128x128, TILE_256x256, TILE_320x224, TILE_288x224 = (
    -1, 0, 1, 2, 3, 4, 5, 6)

EXPORTS = [
    "ocg_config_default", "ocg_create", "ocg_destroy", "ocg_workspace_bytes", "ocg_workspace_bytes_for",
    "ocg_workspace_init", "ocg_ag_gemm", "ocg_gemm_rs", "ocg_ag_grouped_gemm",
    "ocg_signal", "ocg_check", "ocg_status_string", "ocg_plan_info", "ocg_plan_task",
    "ocg_moe_combine_rs", "ocg_ag_attention", "ocg_plan_ag", "ocg_ag_gemm_noalloc",
    "ocg_gemm_rs_push", "ocg_ag_moe_layer",
]


class Config(C.Structure):
    _fields_ = [
        ("tile", C.c_int32), ("slab_rows", C.c_int32), ("copy_rows", C.c_int32),
        ("swizzle", C.c_int32), ("mode", C.c_int32), ("grid", C.c_int32),
        ("spin_timeout_us", C.c_uint32), ("fault_skip_slab", C.c_int32),
        ("trace", C.c_void_p), ("trace_capacity", C.c_uint32),
        ("peer_flags", C.c_void_p), ("peer_flag_value", C.c_uint32),
        ("transfer", C.c_int32), ("kslab_cols", C.c_int32), ("copy_delay", C.c_uint32),
        ("xcd_remap", C.c_int32), ("side_grid", C.c_int32), ("split_k", C.c_int32),
    ]


class TraceRec(C.Structure):
    _fields_ = [
        ("ticket", C.c_uint32), ("kind", C.c_uint32), ("a", C.c_uint32), ("b", C.c_uint32),
        ("c", C.c_uint32), ("d", C.c_uint32), ("hw", C.c_uint32), ("epoch", C.c_uint32),
        ("t_start", C.c_uint64), ("t_ready", C.c_uint64), ("t_end", C.c_uint64),
        ("flag_seen", C.c_uint32), ("queue", C.c_uint32), ("cycles", C.c_uint64),
        ("wait_ticks", C.c_uint32), ("pad", C.c_uint32),
    ]


assert C.sizeof(TraceRec) == 80

I64x8 = C.c_int64 * 8
_P = C.c_void_p


def _declare(lib):
    sig = {
        "ocg_config_default": (None, [C.POINTER(Config)]),
        "ocg_create": (C.c_int, [C.c_int, C.POINTER(C.c_void_p)]),
        "ocg_destroy": (None, [_P]),
        "ocg_workspace_bytes": (C.c_size_t, [_P, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int]),
        "ocg_workspace_bytes_for": (C.c_size_t, [_P, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int,
                                                 _P]),
        "ocg_workspace_init": (C.c_int, [_P, _P, C.c_size_t, _P]),
        "ocg_ag_gemm": (C.c_int, [_P, C.POINTER(_P), C.c_int, C.c_int, C.c_int64, C.c_int64, _P, C.c_int64,
                                  _P, _P, _P, C.c_size_t, C.POINTER(Config), _P]),
        "ocg_ag_gemm_noalloc": (C.c_int, [_P, C.POINTER(_P), C.c_int, C.c_int, C.c_int64, C.c_int64, _P,
                                          C.c_int64, _P, _P, C.POINTER(Config), _P]),
        "ocg_gemm_rs": (C.c_int, [_P, _P, _P, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int,
                                  C.POINTER(_P), _P, _P, _P, C.c_size_t, C.POINTER(Config), _P]),
        "ocg_ag_moe_layer": (C.c_int, [_P, C.POINTER(_P), C.c_int, C.c_int, C.c_int64, C.c_int64, _P,
                                       C.c_int, C.c_int, _P, C.c_int64, C.POINTER(_P), _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P, C.c_size_t, C.POINTER(Config), _P]),
        "ocg_gemm_rs_push": (C.c_int, [_P, _P, _P, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int,
                                       C.POINTER(_P), C.POINTER(_P), C.c_uint32, _P, _P, C.c_size_t,
                                       C.POINTER(Config), _P]),
        "ocg_ag_grouped_gemm": (C.c_int, [_P, C.POINTER(_P), C.c_int, C.c_int, C.c_int64, C.c_int64, _P,
                                          C.c_int, C.c_int, _P, C.c_int64, _P, _P, _P, _P, _P, _P, _P,
                                          C.c_size_t, C.POINTER(Config), _P]),
        "ocg_moe_combine_rs": (C.c_int, [_P, _P, _P, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int, C.POINTER(_P),
                                         _P, _P,
                                         _P, C.c_size_t, C.POINTER(Config), _P]),
        "ocg_ag_attention": (C.c_int, [_P, _P, C.POINTER(_P), C.POINTER(_P), C.c_int, C.c_int, C.c_int64,
                                       C.c_int64, C.c_int64, C.c_int64, _P, _P, _P, _P, C.c_size_t,
                                       C.POINTER(Config), _P]),
        "ocg_signal": (C.c_int, [_P, C.c_int, C.c_uint32, _P]),
        "ocg_check": (C.c_int, [_P, _P]),
        "ocg_status_string": (C.c_char_p, [C.c_int]),
        "ocg_plan_info": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                    C.c_int, C.c_int, C.POINTER(Config), I64x8]),
        "ocg_plan_ag": (C.c_int, [_P, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                  C.POINTER(Config), I64x8]),
        "ocg_plan_task": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                    C.POINTER(Config), C.c_int64, I64x8]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args


def load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python communication_overlapped_gemm_amd/build.py); there is no fallback path")
    lib = C.CDLL(path)
    _declare(lib)
    return lib


lib = load()


def default_config(**kw) -> Config:
    c = Config()
    lib.ocg_config_default(C.byref(c))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def status_string(code: int) -> str:
    return lib.ocg_status_string(code).decode()


class OcgError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


def check(code: int, what: str) -> None:
    if code != OK:
        raise OcgError(code, what)
