"""ctypes loader for libqlora_amd.so (built in-tree by build.py).

There is no fallback: if the library is missing or fails to load, every call
raises. All arithmetic of the hot path runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlora_amd.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "qlora_amd.h")

OK = 0
DTYPE_F32 = 0
DTYPE_BF16 = 1
LAYOUT_ROWS = 0
LAYOUT_KSLAB32 = 1
DQ_INT8 = 0
DQ_UINT8 = 1
DQ_E4M3 = 2
OP_FWD = 0
OP_BWD = 1
OP_MERGE = 2
OP_FWD_LEAN = 3
OP_BWD_LEAN = 4
NOALLOC_SCRATCH_BYTES = 32 << 20

P = ctypes.c_void_p
I64 = ctypes.c_int64
INT = ctypes.c_int
SZ = ctypes.c_size_t
FLT = ctypes.c_float
DBL = ctypes.c_double

class NF4Desc(ctypes.Structure):
    """struct qlora_nf4 of include/qlora_amd.h."""
    _fields_ = [("N", I64), ("K", I64), ("codes", P), ("absmax_q", P), ("absmax_scale", P),
                ("dq_format", ctypes.c_int32), ("format_version", ctypes.c_uint32),
                ("setup_id", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


DESC = ctypes.POINTER(NF4Desc)
FORMAT_VERSION = 1

SIGNATURES = {
    "qlora_strerror": (ctypes.c_char_p, [INT]),
    "qlora_nf4_sizes": (INT, [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
    "qlora_codebook": (INT, [P, P]),
    "qlora_codebook_quotient_thresholds": (INT, [P]),
    "qlora_codebook_id": (ctypes.c_uint32, []),
    "qlora_workspace_bytes": (SZ, [INT, I64, I64, I64, INT]),
    "qlora_setup_id": (ctypes.c_uint32, [INT]),
    "qlora_nf4_check": (INT, [DESC]),
    "qlora_quantize_nf4_dq": (INT, [P, INT, I64, I64, INT, DESC, P]),
    "qlora_dequant_bf16": (INT, [DESC, P, INT, P]),
    "qlora_linear_fwd": (INT, [DESC, P, I64, P, P, INT, FLT, P, INT, P, P, SZ, P]),
    "qlora_linear_bwd": (INT, [DESC, P, P, I64, P, P, INT, FLT, P, P, INT, P, P, INT, P, SZ, P]),
    "qlora_linear_fwd_noalloc": (INT, [DESC, P, I64, P, P, INT, FLT, P, INT, P, P]),
    "qlora_gemm_bf16_nt": (INT, [P, I64, P, I64, INT, P, P, I64, I64, I64, INT, P, INT, P]),
    "qlora_merge_lora": (INT, [DESC, P, I64, I64, P, P, INT, FLT, P, P, SZ, P]),
    "qlora_adamw_step": (INT, [P, P, INT, P, P, P, I64, DBL, DBL, DBL, DBL, DBL, I64, P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m qlora_fine_tuning_blockwise_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/qlora_amd.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_\w+)\s*\(", text)))


def strerror(status: int) -> str:
    return load().qlora_strerror(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        raise RuntimeError(f"{what} failed: {strerror(status)} (status {status})")
