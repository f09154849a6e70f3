"""MI355X-native tiled-matmul hot path: dense Y = X W^T, causal attention
scores and their causal softmax, as hand-written gfx950 HIP kernels behind a C
ABI (``include/cas.h``).

This module is the thin binding: it marshals torch tensors (device memory and
the current HIP stream) into the C ABI of ``libcas.so`` and raises on a
non-zero status. Every step of the computation runs in the HIP kernels; there
is no CPU fallback, and the calls raise if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcas.so")

CAS_F32, CAS_BF16, CAS_F16 = 0, 1, 2
STATUS = {0: "CAS_OK", -1: "CAS_ERR_NULL", -2: "CAS_ERR_SHAPE", -3: "CAS_ERR_DTYPE",
          -4: "CAS_ERR_ALIAS", -5: "CAS_ERR_DEVICE", -6: "CAS_ERR_HIP", -7: "CAS_ERR_UNSUPPORTED",
          -8: "CAS_ERR_MODE"}
SOFTMAX_MODE = {"log": 0, "prob": 1}
EXPORTS = ("cas_gemm_nt", "cas_batch_matmul_nt", "cas_trimul_causal", "cas_causal_row_stats", "cas_causal_softmax",
           "cas_causal_softmax_fused", "cas_causal_attention", "cas_causal_attention_fused", "cas_status_string",
           "cas_last_hip_error", "cas_version")

_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class CasError(RuntimeError):
    def __init__(self, op: str, status: int, message: str):
        super().__init__(f"{op}: {STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.cas_gemm_nt.argtypes = [_vp, _vp, _vp] + [_i64] * 6 + [ctypes.c_int, ctypes.c_int, _vp]
        L.cas_gemm_nt.restype = ctypes.c_int
        L.cas_batch_matmul_nt.argtypes = [_vp, _vp, _vp] + [_i64] * 10 + [ctypes.c_int, ctypes.c_int, _vp]
        L.cas_batch_matmul_nt.restype = ctypes.c_int
        L.cas_trimul_causal.argtypes = [_vp, _vp] + [_i64] * 4 + [ctypes.c_int, ctypes.c_int, _vp]
        L.cas_trimul_causal.restype = ctypes.c_int
        L.cas_causal_row_stats.argtypes = [_vp, _vp, _vp] + [_i64] * 4 + [ctypes.c_int, _vp]
        L.cas_causal_row_stats.restype = ctypes.c_int
        L.cas_causal_softmax.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 4 + [ctypes.c_int] * 3 + [_vp]
        L.cas_causal_softmax.restype = ctypes.c_int
        L.cas_causal_softmax_fused.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 4 + [ctypes.c_int] * 3 + [_vp]
        L.cas_causal_softmax_fused.restype = ctypes.c_int
        L.cas_causal_attention.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 4 + [ctypes.c_int] * 2 + [_vp]
        L.cas_causal_attention.restype = ctypes.c_int
        L.cas_causal_attention_fused.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 4 + [ctypes.c_int] * 2 + [_vp]
        L.cas_causal_attention_fused.restype = ctypes.c_int
        L.cas_status_string.argtypes = [ctypes.c_int]
        L.cas_status_string.restype = ctypes.c_char_p
        L.cas_last_hip_error.restype = ctypes.c_int
        L.cas_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().cas_status_string(status).decode()


def _check(op: str, status: int) -> None:
    if status != 0:
        msg = status_string(status)
        if status in (-5, -6):
            msg += f" (hipError {lib().cas_last_hip_error()})"
        raise CasError(op, status, msg)


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: CAS_F32, torch.bfloat16: CAS_BF16, torch.float16: CAS_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported input dtype {t.dtype}")
    return codes[t.dtype]


def _stream_ptr(dev) -> int:
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _require_device(*ts) -> None:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must live on the same GPU")


def gemm_nt(x, w, out=None):
    """Y = x @ w.T with fp32 accumulation and fp32 output.

    x: [M, K] and w: [N, K] of one dtype (float32, bfloat16, float16), rows
    contiguous (any row pitch); out: optional [M, N] float32 with contiguous
    rows. The kernel runs on the current stream of x's device."""
    import torch
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("gemm_nt expects x [M, K] and w [N, K]")
    if x.dtype != w.dtype:
        raise TypeError("x and w must share a dtype")
    if x.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("rows of x and w must be contiguous")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a float32 [M, N] tensor with contiguous rows")
    _require_device(x, w, out)
    ldx = x.stride(0) if M > 1 else K
    ldw = w.stride(0) if N > 1 else K
    ldy = out.stride(0) if M > 1 else N
    st = lib().cas_gemm_nt(x.data_ptr(), w.data_ptr(), out.data_ptr(), M, N, K, ldx, ldw, ldy,
                           _dtype_code(x), CAS_F32, _stream_ptr(x.device))
    _check("cas_gemm_nt", st)
    return out


def batch_matmul_nt(x, w, out=None):
    """Y[b] = x[b] @ w[b].T for every b, fp32 accumulation and output.

    x: [batch, M, K] and w: [batch, N, K] of one dtype (float32, bfloat16,
    float16), rows contiguous (any row pitch and batch stride; a batch stride
    of 0, as from expand(), repeats one block); out: optional [batch, M, N]
    float32 with contiguous rows. Runs on the current stream of x's device."""
    import torch
    if x.dim() != 3 or w.dim() != 3 or x.shape[0] != w.shape[0] or x.shape[2] != w.shape[2]:
        raise ValueError("batch_matmul_nt expects x [batch, M, K] and w [batch, N, K]")
    if x.dtype != w.dtype:
        raise TypeError("x and w must share a dtype")
    if x.stride(2) != 1 or w.stride(2) != 1:
        raise ValueError("rows of x and w must be contiguous")
    Bt, M, K = x.shape
    N = w.shape[1]
    if out is None:
        out = torch.empty((Bt, M, N), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (Bt, M, N) or (N > 1 and out.stride(2) != 1):
        raise ValueError("out must be a float32 [batch, M, N] tensor with contiguous rows")
    _require_device(x, w, out)
    ldx = x.stride(1) if M > 1 else K
    ldw = w.stride(1) if N > 1 else K
    ldy = out.stride(1) if M > 1 else N
    st = lib().cas_batch_matmul_nt(x.data_ptr(), w.data_ptr(), out.data_ptr(), Bt, M, N, K, ldx, ldw, ldy,
                                   x.stride(0), w.stride(0), out.stride(0), _dtype_code(x), CAS_F32,
                                   _stream_ptr(x.device))
    _check("cas_batch_matmul_nt", st)
    return out


def _qkv_dims(qkv, NH: int):
    """(B, T, C) of a contiguous packed QKV tensor, (B, T, 3C) or (B, T, 3, NH, HS)."""
    if not qkv.is_contiguous():
        raise ValueError("qkv must be contiguous")
    if qkv.dim() == 5:
        B, T, three, nh, HS = qkv.shape
        if three != 3 or nh != NH:
            raise ValueError("qkv must be (B, T, 3, NH, HS)")
        return B, T, NH * HS
    if qkv.dim() == 3:
        B, T, C3 = qkv.shape
        if C3 % 3:
            raise ValueError("last dim of qkv must be 3*C")
        return B, T, C3 // 3
    raise ValueError("qkv must be (B, T, 3C) or (B, T, 3, NH, HS)")


def causal_row_stats(qkv, NH: int, row_max=None, row_logsum=None):
    """Per-row statistics of the causal scores (the row_stats launch of the
    two-launch softmax): row_max[b, nh, t] = max over t2 <= t of the fp32
    score, row_logsum = ln sum exp(score - row_max), both float32 (B, NH, T).
    The scores are recomputed from qkv and never written."""
    import torch
    B, T, C = _qkv_dims(qkv, NH)
    shape = (B, NH, T)
    if row_max is None:
        row_max = torch.empty(shape, dtype=torch.float32, device=qkv.device)
    if row_logsum is None:
        row_logsum = torch.empty(shape, dtype=torch.float32, device=qkv.device)
    for t in (row_max, row_logsum):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("row_max / row_logsum must be contiguous float32 (B, NH, T) tensors")
    _require_device(qkv, row_max, row_logsum)
    st = lib().cas_causal_row_stats(qkv.data_ptr(), row_max.data_ptr(), row_logsum.data_ptr(), B, T, C, NH,
                                    _dtype_code(qkv), _stream_ptr(qkv.device))
    _check("cas_causal_row_stats", st)
    return row_max, row_logsum


def causal_softmax(qkv, NH: int, mode: str = "prob", out=None, out_dtype=None, stats=None, fused=None):
    """Causal softmax of the scores. mode "prob": probabilities, 0 above the
    diagonal; "log": log-probabilities (x - row_max) - row_logsum, -inf above
    it. out_dtype (or out's dtype): float32 (default), bfloat16 or float16.
    stats: an optional (row_max, row_logsum) pair to use as given (the
    softmax-rows launch alone). Without stats, fused=True computes statistics
    and rows in one launch, fused=False in the two launches of row statistics
    then softmax rows; the default (None) takes the one launch for 16-bit
    inputs and the two launches for fp32 inputs, the faster of the two for
    each as measured (both meet the same accuracy bounds; row_max is the
    same, row_logsum may differ in its last bits). Returns (out, row_max,
    row_logsum)."""
    import torch
    if mode not in SOFTMAX_MODE:
        raise ValueError("mode must be 'prob' or 'log'")
    B, T, C = _qkv_dims(qkv, NH)
    if fused is None:
        fused = qkv.dtype != torch.float32
    if stats is None and fused:
        if out is None:
            out = torch.empty((B, NH, T, T), dtype=out_dtype or torch.float32, device=qkv.device)
        if out_dtype is not None and out.dtype != out_dtype:
            raise TypeError("out does not have out_dtype")
        if tuple(out.shape) != (B, NH, T, T) or not out.is_contiguous():
            raise ValueError("out must be a contiguous (B, NH, T, T) tensor")
        row_max = torch.empty((B, NH, T), dtype=torch.float32, device=qkv.device)
        row_logsum = torch.empty((B, NH, T), dtype=torch.float32, device=qkv.device)
        _require_device(qkv, out)
        st = lib().cas_causal_softmax_fused(qkv.data_ptr(), out.data_ptr(), row_max.data_ptr(),
                                            row_logsum.data_ptr(), B, T, C, NH, SOFTMAX_MODE[mode],
                                            _dtype_code(qkv), _dtype_code(out), _stream_ptr(qkv.device))
        _check("cas_causal_softmax_fused", st)
        return out, row_max, row_logsum
    row_max, row_logsum = stats if stats is not None else causal_row_stats(qkv, NH)
    if out is None:
        out = torch.empty((B, NH, T, T), dtype=out_dtype or torch.float32, device=qkv.device)
    if out_dtype is not None and out.dtype != out_dtype:
        raise TypeError("out does not have out_dtype")
    if tuple(out.shape) != (B, NH, T, T) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, NH, T, T) tensor")
    for t in (row_max, row_logsum):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, NH, T) or not t.is_contiguous():
            raise ValueError("row_max / row_logsum must be contiguous float32 (B, NH, T) tensors")
    _require_device(qkv, out, row_max, row_logsum)
    st = lib().cas_causal_softmax(qkv.data_ptr(), row_max.data_ptr(), row_logsum.data_ptr(), out.data_ptr(),
                                  B, T, C, NH, SOFTMAX_MODE[mode], _dtype_code(qkv), _dtype_code(out),
                                  _stream_ptr(qkv.device))
    _check("cas_causal_softmax", st)
    return out, row_max, row_logsum


def causal_attention(qkv, NH: int, y=None, stats=None):
    """Attention output y (B, T, C) float32: the causal softmax probabilities
    times the value rows, per head. stats: an optional (row_max, row_logsum)
    pair, read as given (cas_causal_attention); without it, y and the
    statistics come from the single-pass kernel (cas_causal_attention_fused).
    Returns (y, row_max, row_logsum)."""
    import torch
    if stats is None:
        return causal_attention_fused(qkv, NH, y=y)
    B, T, C = _qkv_dims(qkv, NH)
    row_max, row_logsum = stats
    for t in (row_max, row_logsum):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, NH, T) or not t.is_contiguous():
            raise ValueError("row_max / row_logsum must be contiguous float32 (B, NH, T) tensors")
    if y is None:
        y = torch.empty((B, T, C), dtype=torch.float32, device=qkv.device)
    if y.dtype != torch.float32 or tuple(y.shape) != (B, T, C) or not y.is_contiguous():
        raise ValueError("y must be a contiguous float32 (B, T, C) tensor")
    _require_device(qkv, y, row_max, row_logsum)
    st = lib().cas_causal_attention(qkv.data_ptr(), row_max.data_ptr(), row_logsum.data_ptr(), y.data_ptr(),
                                    B, T, C, NH, _dtype_code(qkv), CAS_F32, _stream_ptr(qkv.device))
    _check("cas_causal_attention", st)
    return y, row_max, row_logsum


def causal_attention_fused(qkv, NH: int, y=None, row_max=None, row_logsum=None):
    """The attention output y (B, T, C) float32 and the row statistics
    (B, NH, T) in one pass (running maximum and sum, y rescaled as they move).
    Returns (y, row_max, row_logsum)."""
    import torch
    B, T, C = _qkv_dims(qkv, NH)
    if y is None:
        y = torch.empty((B, T, C), dtype=torch.float32, device=qkv.device)
    if y.dtype != torch.float32 or tuple(y.shape) != (B, T, C) or not y.is_contiguous():
        raise ValueError("y must be a contiguous float32 (B, T, C) tensor")
    shape = (B, NH, T)
    if row_max is None:
        row_max = torch.empty(shape, dtype=torch.float32, device=qkv.device)
    if row_logsum is None:
        row_logsum = torch.empty(shape, dtype=torch.float32, device=qkv.device)
    for t in (row_max, row_logsum):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("row_max / row_logsum must be contiguous float32 (B, NH, T) tensors")
    _require_device(qkv, y, row_max, row_logsum)
    st = lib().cas_causal_attention_fused(qkv.data_ptr(), y.data_ptr(), row_max.data_ptr(), row_logsum.data_ptr(),
                                          B, T, C, NH, _dtype_code(qkv), CAS_F32, _stream_ptr(qkv.device))
    _check("cas_causal_attention_fused", st)
    return y, row_max, row_logsum


def trimul_causal(qkv, NH: int, out=None, out_dtype=None):
    """Causal attention scores from packed QKV.

    qkv: contiguous (B, T, 3*C) or (B, T, 3, NH, HS) tensor (float32,
    bfloat16 or float16); returns out (B, NH, T, T) with scale * Q.K on and
    below the diagonal and NaN above it. out_dtype (or out's dtype): float32
    (default), or bfloat16 / float16 for the fp32 scores rounded to that
    format (half the output bytes)."""
    import torch
    B, T, C = _qkv_dims(qkv, NH)
    if out is None:
        out = torch.empty((B, NH, T, T), dtype=out_dtype or torch.float32, device=qkv.device)
    if out_dtype is not None and out.dtype != out_dtype:
        raise TypeError("out does not have out_dtype")
    if tuple(out.shape) != (B, NH, T, T) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, NH, T, T) tensor")
    _require_device(qkv, out)
    st = lib().cas_trimul_causal(qkv.data_ptr(), out.data_ptr(), B, T, C, NH,
                                 _dtype_code(qkv), _dtype_code(out), _stream_ptr(qkv.device))
    _check("cas_trimul_causal", st)
    return out
