"""QLoRA frozen-base hot path for MI355X (gfx950): blockwise NF4 quantization
with double quantization, dequantization to bf16, and the QLoRA linear layer
(forward and backward), as hand-written HIP kernels behind a C ABI.

The functions below carry the names of the C entry points
(include/qlora_amd.h). They only marshal arguments: torch supplies device
memory and the current stream, and every step of the computation runs in
libqlora_amd.so. Tensors must be contiguous and on a ROCm device.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib

__all__ = [
    "qlora_strerror", "qlora_nf4_sizes", "qlora_codebook", "qlora_codebook_quotient_thresholds",
    "qlora_codebook_id", "qlora_setup_id", "qlora_nf4_check",
    "qlora_workspace_bytes", "qlora_quantize_nf4_dq", "qlora_dequant_bf16",
    "qlora_linear_fwd", "qlora_linear_bwd", "qlora_linear_fwd_noalloc", "qlora_gemm_bf16_nt", "qlora_merge_lora", "qlora_adamw_step",
    "NF4Weight", "DQ_INT8", "DQ_UINT8", "DQ_E4M3", "LAYOUT_ROWS", "LAYOUT_KSLAB32",
]


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtypes, device):
    """Checks one tensor argument before its pointer crosses the C ABI (the
    library cannot see buffer sizes): shape, dtype, contiguity and device."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return _lib.DTYPE_F32
    if dt == torch.bfloat16:
        return _lib.DTYPE_BF16
    raise ValueError(f"unsupported dtype {dt}")


DQ_INT8, DQ_UINT8, DQ_E4M3 = _lib.DQ_INT8, _lib.DQ_UINT8, _lib.DQ_E4M3
LAYOUT_ROWS, LAYOUT_KSLAB32 = _lib.LAYOUT_ROWS, _lib.LAYOUT_KSLAB32


class NF4Weight:
    """A quantized [N, K] weight: its three device buffers and the metadata of
    the C descriptor (struct qlora_nf4): the second-level format of the
    absmax codes (DQ_INT8, DQ_UINT8, DQ_E4M3), the storage format version and
    the setup id of the library that quantized it. qlora_quantize_nf4_dq
    fills the metadata; a weight restored from storage carries the stored
    values, and the library rejects it if they do not match its own."""

    def __init__(self, codes, absmax_q, absmax_scale, N: int, K: int, dq_format: int = DQ_INT8,
                 format_version: int = 0, setup_id: int = 0):
        self.codes, self.absmax_q, self.absmax_scale = codes, absmax_q, absmax_scale
        self.N, self.K = int(N), int(K)
        self.dq_format = int(dq_format)
        self.format_version = int(format_version)
        self.setup_id = int(setup_id)

    def nbytes(self) -> int:
        return self.codes.numel() + self.absmax_q.numel() + 4 * self.absmax_scale.numel()

    @property
    def device(self):
        return self.codes.device

    def _check_buffers(self):
        cb, qb, sb = qlora_nf4_sizes(self.N, self.K)
        dev = self.codes.device
        _need(self.codes, "codes", (cb,), torch.uint8, dev)
        _need(self.absmax_q, "absmax_q", (qb,), torch.int8, dev)
        _need(self.absmax_scale, "absmax_scale", (sb // 4,), torch.float32, dev)

    def desc(self) -> "ctypes.pointer":
        """The C descriptor of this weight (buffers checked first)."""
        self._check_buffers()
        d = _lib.NF4Desc(self.N, self.K, self.codes.data_ptr(), self.absmax_q.data_ptr(),
                         self.absmax_scale.data_ptr(), self.dq_format, self.format_version,
                         self.setup_id, 0)
        return ctypes.pointer(d)


def qlora_strerror(status: int) -> str:
    return _lib.strerror(status)


def qlora_nf4_sizes(N: int, K: int):
    cb, qb, sb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(_lib.load().qlora_nf4_sizes(N, K, ctypes.byref(cb), ctypes.byref(qb),
                                           ctypes.byref(sb)), "qlora_nf4_sizes")
    return cb.value, qb.value, sb.value


def qlora_codebook():
    lv = np.zeros(16, np.float32)
    th = np.zeros(15, np.float32)
    _lib.check(_lib.load().qlora_codebook(lv.ctypes.data_as(ctypes.c_void_p),
                                          th.ctypes.data_as(ctypes.c_void_p)), "qlora_codebook")
    return lv, th


def qlora_codebook_quotient_thresholds():
    tq = np.zeros(15, np.float32)
    _lib.check(_lib.load().qlora_codebook_quotient_thresholds(tq.ctypes.data_as(ctypes.c_void_p)),
               "qlora_codebook_quotient_thresholds")
    return tq


def qlora_nf4_check(w: NF4Weight) -> int:
    """Status of the library's host check of w's descriptor (0 = usable)."""
    return int(_lib.load().qlora_nf4_check(w.desc()))


def qlora_setup_id(dq_format: int) -> int:
    return int(_lib.load().qlora_setup_id(int(dq_format)))


def qlora_codebook_id() -> int:
    return int(_lib.load().qlora_codebook_id())


def qlora_workspace_bytes(op: int, M: int, N: int, K: int, r: int) -> int:
    return int(_lib.load().qlora_workspace_bytes(op, M, N, K, r))


def _alloc_nf4(N, K, device):
    cb, qb, sb = qlora_nf4_sizes(N, K)
    return (torch.empty(cb, dtype=torch.uint8, device=device),
            torch.empty(qb, dtype=torch.int8, device=device),
            torch.empty(sb // 4, dtype=torch.float32, device=device))


def qlora_quantize_nf4_dq(W: torch.Tensor, out: NF4Weight | None = None, stream=None,
                          dq_format: int | None = None) -> NF4Weight:
    """Quantize a [N, K] fp32 or bf16 device tensor to NF4 + double-quantized
    constants in second-level format dq_format (default: out's format, else
    DQ_INT8). The returned weight carries the descriptor metadata the library
    wrote."""
    if W.dim() != 2:
        raise ValueError("qlora_quantize_nf4_dq: W must be [N, K]")
    N, K = W.shape
    _need(W, "W", (N, K), (torch.float32, torch.bfloat16), W.device)
    if dq_format is None:
        dq_format = out.dq_format if out is not None else DQ_INT8
    if out is None:
        out = NF4Weight(*_alloc_nf4(N, K, W.device), N, K, dq_format)
    if (out.N, out.K) != (N, K):
        raise ValueError("qlora_quantize_nf4_dq: out has another shape")
    out.dq_format = int(dq_format)
    d = out.desc()
    st = _lib.load().qlora_quantize_nf4_dq(_ptr(W), _dtype_code(W.dtype), N, K, out.dq_format, d,
                                           _stream(stream))
    _lib.check(st, "qlora_quantize_nf4_dq")
    out.format_version, out.setup_id = int(d.contents.format_version), int(d.contents.setup_id)
    return out


def qlora_dequant_bf16(w: NF4Weight, out: torch.Tensor | None = None, stream=None,
                       layout: int = LAYOUT_ROWS) -> torch.Tensor:
    """w_hat as bf16: [N, K] (LAYOUT_ROWS) or [K/32, N, 32] (LAYOUT_KSLAB32)."""
    shape = (w.N, w.K) if layout == LAYOUT_ROWS else (w.K // 32, w.N, 32)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=w.device)
    if out.numel() != w.N * w.K:
        raise ValueError("qlora_dequant_bf16: out must hold N*K elements")
    _need(out, "out", tuple(out.shape), torch.bfloat16, w.device)
    st = _lib.load().qlora_dequant_bf16(w.desc(), _ptr(out), int(layout), _stream(stream))
    _lib.check(st, "qlora_dequant_bf16")
    return out


def _workspace(op, M, N, K, r, device, workspace):
    need = qlora_workspace_bytes(op, M, N, K, r)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous() \
            or workspace.device != device:
        raise ValueError("workspace: a contiguous 1-D uint8 tensor on the weight's device")
    return workspace


def qlora_linear_fwd(w: NF4Weight, x: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                     alpha: float, y: torch.Tensor | None = None, y_dtype=torch.float32,
                     u_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None, lean: bool = False) -> torch.Tensor:
    """y = x W_hat^T + (alpha/r) (x A) B. x [M,K] bf16, A [K,r] bf16, B [r,N] bf16.
    The route follows the workspace size (an allocated one is sized for the
    fast route, or for the lean route that holds no bf16 copy of the weight
    when `lean`)."""
    M = x.shape[0]
    r = A.shape[1]
    dev = w.device
    _need(x, "x", (M, w.K), torch.bfloat16, dev)
    _need(A, "A", (w.K, r), torch.bfloat16, dev)
    _need(B, "B", (r, w.N), torch.bfloat16, dev)
    if y is None:
        y = torch.empty((M, w.N), dtype=y_dtype, device=dev)
    _need(y, "y", (M, w.N), (torch.float32, torch.bfloat16), dev)
    _need(u_out, "u_out", (M, r), torch.float32, dev)
    workspace = _workspace(_lib.OP_FWD_LEAN if lean else _lib.OP_FWD, M, w.N, w.K, r, dev,
                           workspace)
    st = _lib.load().qlora_linear_fwd(
        w.desc(), _ptr(x), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(y), _dtype_code(y.dtype),
        _ptr(u_out), _ptr(workspace), workspace.numel(), _stream(stream))
    _lib.check(st, "qlora_linear_fwd")
    return y


def qlora_linear_fwd_noalloc(w: NF4Weight, x: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             alpha: float, y: torch.Tensor, u_out: torch.Tensor | None = None,
                             stream=None) -> torch.Tensor:
    """qlora_linear_fwd with the library's own device array as the workspace:
    the call allocates nothing (y and u_out are the caller's)."""
    M = x.shape[0]
    r = A.shape[1]
    dev = w.device
    _need(x, "x", (M, w.K), torch.bfloat16, dev)
    _need(A, "A", (w.K, r), torch.bfloat16, dev)
    _need(B, "B", (r, w.N), torch.bfloat16, dev)
    _need(y, "y", (M, w.N), (torch.float32, torch.bfloat16), dev)
    _need(u_out, "u_out", (M, r), torch.float32, dev)
    st = _lib.load().qlora_linear_fwd_noalloc(
        w.desc(), _ptr(x), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(y), _dtype_code(y.dtype),
        _ptr(u_out), _stream(stream))
    _lib.check(st, "qlora_linear_fwd_noalloc")
    return y


def qlora_linear_bwd(w: NF4Weight, x: torch.Tensor | None, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, alpha: float, u_saved: torch.Tensor | None = None,
                     want_dx: bool = True, dx_dtype=torch.float32, grad_dtype=torch.float32,
                     want_grads: bool = True, workspace: torch.Tensor | None = None,
                     stream=None, lean: bool = False):
    """Returns (dX or None, dA or None, dB or None). With lean=True (and no
    workspace given) the call gets the smallest workspace it accepts, so from
    512 rows on dX is computed without a bf16 copy of the weight."""
    M = dY.shape[0]
    r = A.shape[1]
    dev = w.device
    _need(dY, "dY", (M, w.N), torch.bfloat16, dev)
    _need(x, "x", (M, w.K), torch.bfloat16, dev)
    _need(A, "A", (w.K, r), torch.bfloat16, dev)
    _need(B, "B", (r, w.N), torch.bfloat16, dev)
    _need(u_saved, "u_saved", (M, r), torch.float32, dev)
    dX = torch.empty((M, w.K), dtype=dx_dtype, device=dev) if want_dx else None
    dA = torch.empty((w.K, r), dtype=grad_dtype, device=dev) if want_grads else None
    dB = torch.empty((r, w.N), dtype=grad_dtype, device=dev) if want_grads else None
    workspace = _workspace(_lib.OP_BWD_LEAN if lean else _lib.OP_BWD, M, w.N, w.K, r, dev,
                           workspace)
    st = _lib.load().qlora_linear_bwd(
        w.desc(), _ptr(x), _ptr(dY), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(u_saved),
        _ptr(dX), _dtype_code(dx_dtype), _ptr(dA), _ptr(dB), _dtype_code(grad_dtype),
        _ptr(workspace), workspace.numel(), _stream(stream))
    _lib.check(st, "qlora_linear_bwd")
    return dX, dA, dB


def qlora_gemm_bf16_nt(a: torch.Tensor, b: torch.Tensor, e: torch.Tensor, f: torch.Tensor,
                       y: torch.Tensor | None = None, y_dtype=torch.float32,
                       stream=None, b_layout: int = LAYOUT_ROWS) -> torch.Tensor:
    """y = a b^T + e [f|f]^T. a [M,K], b [N,K] (LAYOUT_ROWS) or [K/32,N,32]
    (LAYOUT_KSLAB32), e [M,2r], f [N,r], all bf16."""
    M, K = a.shape
    if b_layout == LAYOUT_ROWS:
        N = b.shape[0]
        b_ok = b.shape == (N, K)
    else:
        N = b.shape[1]
        b_ok = b.shape == (K // 32, N, 32)
    r = f.shape[1]
    if not b_ok or e.shape != (M, 2 * r) or f.shape[0] != N:
        raise ValueError("qlora_gemm_bf16_nt: inconsistent shapes")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=a.device)
    st = _lib.load().qlora_gemm_bf16_nt(_ptr(a), K, _ptr(b), K, int(b_layout), _ptr(e), _ptr(f), M,
                                        N, K, r, _ptr(y), _dtype_code(y.dtype), _stream(stream))
    _lib.check(st, "qlora_gemm_bf16_nt")
    return y


def qlora_merge_lora(A: torch.Tensor, B: torch.Tensor, alpha: float, w: NF4Weight | None = None,
                     W: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """merged = base + (alpha/r) (A B)^T as fp32 [N, K]; base = the dequantized
    NF4 weight w, or the bf16 weight W. Requantize with qlora_quantize_nf4_dq."""
    if (w is None) == (W is None):
        raise ValueError("qlora_merge_lora: give exactly one of w (NF4) and W (bf16)")
    N, K = (w.N, w.K) if w is not None else W.shape
    r = A.shape[1]
    dev = A.device
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=dev)
    need = qlora_workspace_bytes(_lib.OP_MERGE, 0, N, K, r)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(W, "W", (N, K), torch.bfloat16, dev)
    _need(A, "A", (K, r), torch.bfloat16, dev)
    _need(B, "B", (r, N), torch.bfloat16, dev)
    _need(out, "out", (N, K), torch.float32, dev)
    st = _lib.load().qlora_merge_lora(w.desc() if w is not None else None, _ptr(W), N, K,
                                      _ptr(A), _ptr(B), r, float(alpha), _ptr(out),
                                      _ptr(workspace), workspace.numel(), _stream(stream))
    _lib.check(st, "qlora_merge_lora")
    return out



def qlora_adamw_step(param: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor,
                     exp_avg_sq: torch.Tensor, step: int, lr: float, beta1: float = 0.9,
                     beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
                     param_bf16: torch.Tensor | None = None, stream=None) -> None:
    """One AdamW step in place on flat fp32 master values, moments and an
    optional bf16 copy; grad is bf16 or fp32. The arrays may be device tensors
    or pinned host tensors (the paged state); the step runs on the GPU."""
    n = param.numel()
    for name, t, dt in (("param", param, torch.float32), ("exp_avg", exp_avg, torch.float32),
                        ("exp_avg_sq", exp_avg_sq, torch.float32),
                        ("param_bf16", param_bf16, torch.bfloat16)):
        if t is not None and (t.dtype != dt or t.numel() != n):
            raise ValueError(f"qlora_adamw_step: {name} must be {dt} with {n} elements")
    if grad.numel() != n:
        raise ValueError("qlora_adamw_step: grad must have as many elements as param")
    st = _lib.load().qlora_adamw_step(_ptr(param), _ptr(grad), _dtype_code(grad.dtype),
                                      _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(param_bf16), n,
                                      float(lr), float(beta1), float(beta2), float(eps),
                                      float(weight_decay), int(step), _stream(stream))
    _lib.check(st, "qlora_adamw_step")
