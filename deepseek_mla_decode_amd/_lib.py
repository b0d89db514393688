"""ctypes view of ``libmla_decode.so`` (the C ABI declared in include/mla_decode.h)."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
STATUS_NAMES = {0: "MLA_OK", -1: "MLA_ERR_INVALID_ARG", -2: "MLA_ERR_UNSUPPORTED",
                -3: "MLA_ERR_WORKSPACE", -4: "MLA_ERR_HIP"}

MLA_DTYPE_F16 = 0
MLA_DTYPE_BF16 = 1
MLA_KV_AS_DTYPE = 0
MLA_KV_FP8_E4M3 = 1
D_LATENT = 512
D_ROPE = 64
SPLIT_BLOCK_ROWS = 64
MAX_SPLITS = 1024
NOALLOC_SCRATCH_BYTES = 100 << 20


class MlaDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("page_block_size", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("q_nope_sb", ctypes.c_int64), ("q_nope_sh", ctypes.c_int64),
        ("q_pe_sb", ctypes.c_int64), ("q_pe_sh", ctypes.c_int64),
        ("kv_sb", ctypes.c_int64), ("kv_sr", ctypes.c_int64),
        ("kpe_sb", ctypes.c_int64), ("kpe_sr", ctypes.c_int64),
        ("out_sb", ctypes.c_int64), ("out_sh", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("kv_scale", ctypes.c_float),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)

SIGNATURES = {
    "mla_num_cus": (ctypes.c_int, [ctypes.c_int, _PI32]),
    "mla_max_work": (ctypes.c_int, [ctypes.POINTER(MlaDesc), _I32, _I32, _PI32]),
    "mla_workspace_size": (ctypes.c_int, [ctypes.POINTER(MlaDesc), _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_plan_host": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I32]),
    "mla_plan_device": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P]),
    "mla_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P, _P,
                                  ctypes.POINTER(MlaDesc), _P, ctypes.c_size_t, _P]),
    "mla_decode_planned": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _I32, _P, _P,
                                          ctypes.POINTER(MlaDesc), _P, ctypes.c_size_t, _P]),
    "mla_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P, _P,
                                          ctypes.POINTER(MlaDesc), _P]),
    "mla_check_block_table": (ctypes.c_int, [_P, _P, ctypes.POINTER(MlaDesc), _P, _P]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "mla_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), _PI32]),
}


def lib():
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is missing: build it with `python -m deepseek_mla_decode_amd.build` "
                        "(or __graft_entry__.build()); there is no fallback implementation")
                l = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(l, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = l
    return _lib


def check(status: int) -> None:
    if status != MLA_OK:
        raise MlaError(status, lib().mla_last_error().decode(errors="replace"))
