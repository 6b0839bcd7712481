"""Python access to the CPU oracle (oracle.c) through ctypes.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. The GPU library
and its Python binding never import it; the two share no code.

All arrays are numpy arrays. bf16 tensors travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

BLOCK = 64
GROUP = 256

_CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    cmd = ["gcc", *_CFLAGS, SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        sig = {
            "oracle_norm_cdf": (D, [D]),
            "oracle_norm_ppf": (D, [D]),
            "oracle_nf4_levels_f64": (None, [P]),
            "oracle_nf4_codebook": (None, [P, P]),
            "oracle_nf4_code": (ctypes.c_int, [ctypes.c_float]),
            "oracle_nf4_codes_batch": (ctypes.c_int, [P, I64, P]),
            "oracle_quantize_nf4_f32": (ctypes.c_int, [P, I64, P, P]),
            "oracle_double_quant": (ctypes.c_int, [P, I64, P, P]),
            "oracle_quantize_nf4_dq_f32": (ctypes.c_int, [P, I64, P, P, P]),
            "oracle_quantize_nf4_dq_bf16": (ctypes.c_int, [P, I64, P, P, P]),
            "oracle_dequant_dq": (ctypes.c_int, [P, P, P, I64, P, P]),
            "oracle_dequant_nodq": (ctypes.c_int, [P, P, I64, P, P]),
            "oracle_int4_absmax": (ctypes.c_int, [P, I64, I64, P, P, P]),
            "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "oracle_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_lora_down_xa": (ctypes.c_int, [P, I64, I64, P, ctypes.c_int, P]),
            "oracle_lora_down_dybt": (ctypes.c_int, [P, I64, I64, P, ctypes.c_int, P]),
            "oracle_linear_fwd": (ctypes.c_int, [P, I64, I64, P, I64, P, P, ctypes.c_int, D, P, P]),
            "oracle_linear_bwd": (ctypes.c_int,
                                  [P, P, I64, I64, P, I64, P, P, ctypes.c_int, D, P, P, P]),
            "oracle_merge_lora": (ctypes.c_int, [P, P, P, ctypes.c_int, P, I64, I64, P, P,
                                                 ctypes.c_int, ctypes.c_float, P]),
            "oracle_e4m3_to_f32": (ctypes.c_float, [ctypes.c_uint8]),
            "oracle_f32_to_e4m3": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_q8_value": (ctypes.c_float, [ctypes.c_uint8, ctypes.c_int]),
            "oracle_double_quant_fmt": (ctypes.c_int, [P, I64, ctypes.c_int, P, P]),
            "oracle_quantize_nf4_dq_fmt": (ctypes.c_int, [P, ctypes.c_int, I64, ctypes.c_int, P,
                                                          P, P]),
            "oracle_dequant_dq_fmt": (ctypes.c_int, [P, P, P, I64, ctypes.c_int, P, P]),
            "oracle_adamw_step": (ctypes.c_int, [P, P, ctypes.c_int, P, P, I64] +
                                  [D] * 5 + [I64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (status {rc})")


# ---------------------------------------------------------------- codebook
def norm_ppf(p: float) -> float:
    return lib().oracle_norm_ppf(float(p))


def norm_cdf(t: float) -> float:
    return lib().oracle_norm_cdf(float(t))


def nf4_levels_f64() -> np.ndarray:
    out = np.zeros(16, np.float64)
    lib().oracle_nf4_levels_f64(_p(out))
    return out


def nf4_codebook():
    """(levels fp32[16], thresholds fp32[15])."""
    lv = np.zeros(16, np.float32)
    th = np.zeros(15, np.float32)
    lib().oracle_nf4_codebook(_p(lv), _p(th))
    return lv, th


def nf4_codes(x) -> np.ndarray:
    """Threshold-rule code of every fp32 value in x."""
    x = _c(x, np.float32).ravel()
    out = np.zeros(x.size, np.uint8)
    _check(lib().oracle_nf4_codes_batch(_p(x), x.size, _p(out)), "nf4_codes")
    return out


# ---------------------------------------------------------------- quantize
def sizes(n: int):
    """(codes bytes, q8 bytes, s2 count) for n weights."""
    nb = n // BLOCK
    return n // 2, nb, (nb + GROUP - 1) // GROUP


def quantize_nf4_first(w) -> tuple[np.ndarray, np.ndarray]:
    """First level only: (codes uint8[n/2], c1 fp32[n/64]) from fp32 weights."""
    w = _c(w, np.float32).ravel()
    codes = np.zeros(w.size // 2, np.uint8)
    c1 = np.zeros(w.size // BLOCK, np.float32)
    _check(lib().oracle_quantize_nf4_f32(_p(w), w.size, _p(codes), _p(c1)), "quantize_nf4_f32")
    return codes, c1


# Second-level formats of the 8-bit absmax code (the q8 arrays below are
# byte containers of dtype int8 in every format).
DQ_INT8, DQ_UINT8, DQ_E4M3 = 0, 1, 2


def e4m3_to_f32(b) -> np.ndarray:
    """Values of FP8 E4M3 codes (uint8 array)."""
    b = _c(b, np.uint8).ravel()
    return np.array([lib().oracle_e4m3_to_f32(int(x)) for x in b], np.float32)


def f32_to_e4m3(x) -> np.ndarray:
    """Nearest E4M3 codes of non-negative fp32 values (ties to even, saturating)."""
    x = _c(x, np.float32).ravel()
    return np.array([lib().oracle_f32_to_e4m3(float(v)) for v in x], np.uint8)


def double_quant(c1, fmt: int = DQ_INT8):
    c1 = _c(c1, np.float32).ravel()
    nb = c1.size
    q8 = np.zeros(nb, np.int8)
    s2 = np.zeros((nb + GROUP - 1) // GROUP, np.float32)
    _check(lib().oracle_double_quant_fmt(_p(c1), nb, int(fmt), _p(q8), _p(s2)), "double_quant")
    return q8, s2


def quantize_nf4_dq(w, dtype: str, fmt: int = DQ_INT8):
    """Both levels. ``dtype`` is 'f32' (fp32 values) or 'bf16' (uint16 bit
    patterns); ``fmt`` the second-level format.

    Returns (codes uint8[n/2], q8 int8[n/64] (bytes), s2 fp32[ceil(n/16384)]).
    """
    if dtype == "f32":
        w = _c(w, np.float32).ravel()
    elif dtype == "bf16":
        w = _c(w, np.uint16).ravel()
    else:
        raise ValueError(dtype)
    nc, nb, ng = sizes(w.size)
    codes = np.zeros(nc, np.uint8)
    q8 = np.zeros(nb, np.int8)
    s2 = np.zeros(ng, np.float32)
    _check(lib().oracle_quantize_nf4_dq_fmt(_p(w), int(dtype == "bf16"), w.size, int(fmt),
                                            _p(codes), _p(q8), _p(s2)), "quantize_nf4_dq")
    return codes, q8, s2


def dequant_dq(codes, q8, s2, fmt: int = DQ_INT8):
    """(fp32 products, bf16 bit patterns) of every weight."""
    codes = _c(codes, np.uint8).ravel()
    q8 = np.ascontiguousarray(q8).view(np.uint8).ravel()
    s2 = _c(s2, np.float32).ravel()
    n = codes.size * 2
    w32 = np.zeros(n, np.float32)
    wb = np.zeros(n, np.uint16)
    _check(lib().oracle_dequant_dq_fmt(_p(codes), _p(q8), _p(s2), n, int(fmt), _p(w32), _p(wb)),
           "dequant_dq")
    return w32, wb


def dequant_nodq(codes, c1):
    codes = _c(codes, np.uint8).ravel()
    c1 = _c(c1, np.float32).ravel()
    n = codes.size * 2
    w32 = np.zeros(n, np.float32)
    wb = np.zeros(n, np.uint16)
    _check(lib().oracle_dequant_nodq(_p(codes), _p(c1), n, _p(w32), _p(wb)), "dequant_nodq")
    return w32, wb


def int4_absmax(w, block: int):
    """The pages' symmetric int4 quantizer: (q int8, scale fp32 per block, w_hat fp32)."""
    w = _c(w, np.float32).ravel()
    q = np.zeros(w.size, np.int8)
    sc = np.zeros(w.size // block, np.float32)
    wh = np.zeros(w.size, np.float32)
    _check(lib().oracle_int4_absmax(_p(w), w.size, block, _p(q), _p(sc), _p(wh)), "int4_absmax")
    return q, sc, wh


def bf16_to_f32(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(f)))


# ---------------------------------------------------------------- linear layer
def lora_down_xa(x, A, r: int):
    x = _c(x, np.uint16)
    A = _c(A, np.uint16)
    M, K = x.shape
    u = np.zeros((M, r), np.float64)
    _check(lib().oracle_lora_down_xa(_p(x), M, K, _p(A), r, _p(u)), "lora_down_xa")
    return u


def lora_down_dybt(dY, B, r: int):
    dY = _c(dY, np.uint16)
    B = _c(B, np.uint16)
    M, N = dY.shape
    v = np.zeros((M, r), np.float64)
    _check(lib().oracle_lora_down_dybt(_p(dY), M, N, _p(B), r, _p(v)), "lora_down_dybt")
    return v


def linear_fwd(x, What, A, B, r: int, alpha: float, want_y: bool = True):
    """Double-precision forward: returns (y [M,N] or None, u [M,r])."""
    x = _c(x, np.uint16)
    What = _c(What, np.uint16)
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, K = x.shape
    N = What.shape[0]
    y = np.zeros((M, N), np.float64) if want_y else None
    u = np.zeros((M, r), np.float64)
    _check(lib().oracle_linear_fwd(_p(x), M, K, _p(What), N, _p(A), _p(B), r, float(alpha),
                                   _p(y), _p(u)), "linear_fwd")
    return y, u


def linear_bwd(x, dY, What, A, B, r: int, alpha: float, want=("dX", "dA", "dB")):
    """Double-precision backward: returns dict with the requested of dX, dA, dB."""
    dY = _c(dY, np.uint16)
    What = _c(What, np.uint16)
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    x = None if x is None else _c(x, np.uint16)
    M, N = dY.shape
    K = What.shape[1]
    dX = np.zeros((M, K), np.float64) if "dX" in want else None
    dA = np.zeros((K, r), np.float64) if "dA" in want else None
    dB = np.zeros((r, N), np.float64) if "dB" in want else None
    _check(lib().oracle_linear_bwd(_p(x), _p(dY), M, K, _p(What), N, _p(A), _p(B), r,
                                   float(alpha), _p(dX), _p(dA), _p(dB)), "linear_bwd")
    out = {}
    if dX is not None:
        out["dX"] = dX
    if dA is not None:
        out["dA"] = dA
    if dB is not None:
        out["dB"] = dB
    return out


# ------------------------------------------------------------------ merge
def merge_lora(A, B, r: int, alpha: float, nf4=None, W=None):
    """[P1] bullets (merging forces a re-quantization); [P4] "Merge friction".
    out = base + (alpha/r) (A B)^T in binary32 with the adapter sum in order
    j = 0..r-1, one fused multiply-add per term; base = dequantized NF4 (nf4 =
    (codes, q8, s2, N, K[, fmt])) or the bf16 weight W [N, K] (uint16 bits).
    Returns fp32 [N, K]."""
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    if W is not None:
        W = _c(W, np.uint16)
        N, K = W.shape
        codes = q8 = s2 = None
        fmt = DQ_INT8
    else:
        codes, q8, s2, N, K = nf4[:5]
        fmt = nf4[5] if len(nf4) > 5 else DQ_INT8
        codes, q8, s2 = _c(codes, np.uint8), _c(q8, np.int8), _c(s2, np.float32)
    out = np.empty((N, K), np.float32)
    _check(lib().oracle_merge_lora(_p(codes), _p(q8), _p(s2), int(fmt), _p(W), N, K, _p(A), _p(B), r,
                                   float(alpha), _p(out)), "merge_lora")
    return out



# ------------------------------------------------------------------ AdamW
def adamw_step(p, g, m, v, lr: float, beta1: float, beta2: float, eps: float, wd: float,
               t: int):
    """[P2] precision table (fp32 Adam state, 12 bytes per adapter parameter:
    master value and two moments); [P4] "The memory term LoRA does not
    remove". One AdamW step in binary32 on copies of p, m, v (fp32 arrays of
    one shape); g is fp32 or bf16 bits (uint16). Returns (p, m, v, p_bf16)."""
    p = np.array(p, np.float32, copy=True, order="C")
    m = np.array(m, np.float32, copy=True, order="C")
    v = np.array(v, np.float32, copy=True, order="C")
    g = np.ascontiguousarray(g)
    if g.dtype not in (np.float32, np.uint16) or g.shape != p.shape:
        raise ValueError("g must be fp32 or bf16 bits of the parameters' shape")
    if m.shape != p.shape or v.shape != p.shape:
        raise ValueError("m and v must have the parameters' shape")
    pb = np.empty(p.shape, np.uint16)
    _check(lib().oracle_adamw_step(_p(p), _p(g), int(g.dtype == np.uint16), _p(m), _p(v),
                                   p.size, float(lr), float(beta1), float(beta2), float(eps),
                                   float(wd), int(t), _p(pb)), "adamw_step")
    return p, m, v, pb
