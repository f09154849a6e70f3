"""ctypes view of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no
code with the HIP path; the product never imports it.

Inputs are numpy arrays: float32 for fp32, uint16 bit patterns for bfloat16,
float16 (or uint16 bit patterns) for binary16. Outputs are float32 scores (the
softmax: float64) and float64 error bounds (sum of |products|, scaled like the
output).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2}
QNAN_BITS = 0x7FC00000

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class Oracle:
    """One loaded copy of an oracle library (the default one, or a variant)."""

    def __init__(self, path: str | None = None):
        path = path or _build.LIB
        if not os.path.exists(path):
            _build.build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_gemm_nt.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 6 + [ctypes.c_int]
        lib.oracle_trimul_causal.argtypes = [_vp, _vp, _vp] + [_i64] * 4 + [ctypes.c_int]
        lib.oracle_trimul_causal_rows.argtypes = [_vp, _vp, _vp] + [_i64] * 8 + [ctypes.c_int]
        lib.oracle_causal_softmax_rows.argtypes = [_vp] * 5 + [_i64] * 8 + [ctypes.c_int] * 2
        lib.oracle_causal_softmax.argtypes = [_vp] * 5 + [_i64] * 4 + [ctypes.c_int] * 2
        lib.oracle_causal_attention_rows.argtypes = [_vp] * 3 + [_i64] * 7 + [ctypes.c_int]
        lib.oracle_tiled_matmul_count.argtypes = [_vp, _vp, _vp] + [_i64] * 6 + [_vp]
        lib.oracle_decode.argtypes = [_vp, ctypes.c_int, _i64, _vp]
        lib.oracle_round16.argtypes = [_vp, _vp, _i64, ctypes.c_int]
        lib.oracle_trimul_scale.argtypes = [_i64]
        lib.oracle_trimul_scale.restype = ctypes.c_float
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib

    # ---------------------------------------------------------------- utils
    @staticmethod
    def _raw(a: np.ndarray, dtype: str) -> np.ndarray:
        if dtype == "f32":
            return np.ascontiguousarray(a, dtype=np.float32)
        if dtype == "f16" and a.dtype == np.float16:
            return np.ascontiguousarray(a).view(np.uint16)
        if a.dtype != np.uint16:
            raise TypeError(f"{dtype} input must be given as uint16 bit patterns")
        return np.ascontiguousarray(a)

    @staticmethod
    def _p(a: np.ndarray | None):
        return None if a is None else a.ctypes.data_as(_vp)

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(n)

    def decode(self, a: np.ndarray, dtype: str) -> np.ndarray:
        raw = self._raw(a, dtype)
        out = np.empty(raw.size, dtype=np.float64)
        rc = self.lib.oracle_decode(self._p(raw), DTYPE_CODE[dtype], raw.size, self._p(out))
        if rc:
            raise ValueError("oracle_decode rejected its arguments")
        return out.reshape(raw.shape)

    def round16(self, a: np.ndarray, dtype: str) -> np.ndarray:
        """binary32 -> bfloat16 / binary16 bit patterns (uint16), nearest even."""
        src = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(src.shape, dtype=np.uint16)
        rc = self.lib.oracle_round16(self._p(src), self._p(out), src.size, DTYPE_CODE[dtype])
        if rc:
            raise ValueError("oracle_round16 rejected its arguments")
        return out

    def trimul_scale(self, hs: int) -> np.float32:
        return np.float32(self.lib.oracle_trimul_scale(hs))

    # ------------------------------------------------------------- methods
    def gemm_nt(self, X: np.ndarray, W: np.ndarray, dtype: str = "f32", *,
                M=None, N=None, K=None, ldx=None, ldw=None, ldy=None,
                with_bound: bool = True):
        """Y = X W^T. X is [M, ldx] and W is [N, ldw] (2-D arrays), or flat
        buffers with explicit sizes and pitches."""
        rx, rw = self._raw(X, dtype), self._raw(W, dtype)
        if M is None:
            M, K = X.shape
            N = W.shape[0]
            ldx, ldw = X.shape[1], W.shape[1]
        ldy = N if ldy is None else ldy
        Y = np.zeros((M, ldy), dtype=np.float32)
        bound = np.zeros((M, ldy), dtype=np.float64) if with_bound else None
        rc = self.lib.oracle_gemm_nt(self._p(rx), self._p(rw), self._p(Y), self._p(bound),
                                     M, N, K, ldx, ldw, ldy, DTYPE_CODE[dtype])
        if rc:
            raise ValueError("oracle_gemm_nt rejected its arguments")
        return Y, bound

    def batch_matmul_nt(self, X: np.ndarray, W: np.ndarray, dtype: str = "f32", with_bound: bool = True):
        """BatchMatmulNT (DietCode test_1_local_padding.py, test_local_padding_ii
        docstring): Y[i] = X[i] W[i]^T for every batch index i, each block the
        dense product above. X is [batch, M, K], W is [batch, N, K]."""
        Bt, M, K = X.shape
        N = W.shape[1]
        Y = np.zeros((Bt, M, N), dtype=np.float32)
        bound = np.zeros((Bt, M, N), dtype=np.float64) if with_bound else None
        for i in range(Bt):
            y, b = self.gemm_nt(X[i], W[i], dtype, with_bound=with_bound)
            Y[i] = y
            if with_bound:
                bound[i] = b
        return Y, bound

    def trimul_causal(self, qkv: np.ndarray, B: int, T: int, C: int, NH: int,
                      dtype: str = "f32", with_bound: bool = True):
        raw = self._raw(qkv, dtype)
        out = np.empty((B, NH, T, T), dtype=np.float32)
        bound = np.empty((B, NH, T, T), dtype=np.float64) if with_bound else None
        rc = self.lib.oracle_trimul_causal(self._p(raw), self._p(out), self._p(bound),
                                           B, T, C, NH, DTYPE_CODE[dtype])
        if rc:
            raise ValueError("oracle_trimul_causal rejected its arguments")
        return out, bound

    def trimul_causal_rows(self, qkv: np.ndarray, B: int, T: int, C: int, NH: int,
                           b: int, nh: int, t0: int, t1: int, dtype: str = "f32",
                           with_bound: bool = True):
        raw = self._raw(qkv, dtype)
        out = np.empty((t1 - t0, T), dtype=np.float32)
        bound = np.empty((t1 - t0, T), dtype=np.float64) if with_bound else None
        rc = self.lib.oracle_trimul_causal_rows(self._p(raw), self._p(out), self._p(bound),
                                                B, T, C, NH, b, nh, t0, t1, DTYPE_CODE[dtype])
        if rc:
            raise ValueError("oracle_trimul_causal_rows rejected its arguments")
        return out, bound

    SOFTMAX_MODE = {"log": 0, "prob": 1}

    def causal_softmax(self, qkv: np.ndarray, B: int, T: int, C: int, NH: int, dtype: str = "f32",
                       mode: str = "prob", with_out: bool = True, with_bound: bool = True):
        """Causal softmax of the scores (smallem "Kernels GPU", the softmax in
        two launches, over the trimul_cpu score rows). Returns (out (B,NH,T,T)
        or None, row_max (B,NH,T), row_logsum (B,NH,T), bound or None), all
        float64."""
        raw = self._raw(qkv, dtype)
        out = np.empty((B, NH, T, T), dtype=np.float64) if with_out else None
        mx = np.empty((B, NH, T), dtype=np.float64)
        ls = np.empty((B, NH, T), dtype=np.float64)
        bound = np.empty((B, NH, T, T), dtype=np.float64) if with_bound else None
        rc = self.lib.oracle_causal_softmax(self._p(raw), self._p(out), self._p(mx), self._p(ls), self._p(bound),
                                            B, T, C, NH, DTYPE_CODE[dtype], self.SOFTMAX_MODE[mode])
        if rc:
            raise ValueError("oracle_causal_softmax rejected its arguments")
        return out, mx, ls, bound

    def causal_softmax_rows(self, qkv: np.ndarray, B: int, T: int, C: int, NH: int, b: int, nh: int,
                            t0: int, t1: int, dtype: str = "f32", mode: str = "prob",
                            with_out: bool = True, with_bound: bool = True):
        """Rows [t0, t1) of plane (b, nh) of causal_softmax."""
        raw = self._raw(qkv, dtype)
        n = t1 - t0
        out = np.empty((n, T), dtype=np.float64) if with_out else None
        mx = np.empty(n, dtype=np.float64)
        ls = np.empty(n, dtype=np.float64)
        bound = np.empty((n, T), dtype=np.float64) if with_bound else None
        rc = self.lib.oracle_causal_softmax_rows(self._p(raw), self._p(out), self._p(mx), self._p(ls),
                                                 self._p(bound), B, T, C, NH, b, nh, t0, t1,
                                                 DTYPE_CODE[dtype], self.SOFTMAX_MODE[mode])
        if rc:
            raise ValueError("oracle_causal_softmax_rows rejected its arguments")
        return out, mx, ls, bound

    def causal_attention(self, qkv: np.ndarray, B: int, T: int, C: int, NH: int, dtype: str = "f32",
                         with_abs: bool = True, b_range=None, t_range=None):
        """Attention output y (B, T, C) (or batches b_range, rows t_range) of
        the causal softmax times the value rows, float64; with the error
        scale sum p |V| of each output."""
        raw = self._raw(qkv, dtype)
        bs = range(B) if b_range is None else b_range
        t0, t1 = (0, T) if t_range is None else t_range
        y = np.empty((len(bs), t1 - t0, C), dtype=np.float64)
        aw = np.empty((len(bs), t1 - t0, C), dtype=np.float64) if with_abs else None
        for n, b in enumerate(bs):
            rc = self.lib.oracle_causal_attention_rows(self._p(raw), self._p(y[n]), self._p(None if aw is None else aw[n]),
                                                       B, T, C, NH, b, t0, t1, DTYPE_CODE[dtype])
            if rc:
                raise ValueError("oracle_causal_attention_rows rejected its arguments")
        return y, aw

    def tiled_matmul_count(self, A: np.ndarray, Bm: np.ndarray, bm: int, bn: int, bk: int):
        """Returns (A@B, loads, writes, padded_loads, padded_writes)."""
        A = np.ascontiguousarray(A, dtype=np.float32)
        Bm = np.ascontiguousarray(Bm, dtype=np.float32)
        M, K = A.shape
        N = Bm.shape[1]
        out = np.zeros((M, N), dtype=np.float32)
        counts = np.zeros(4, dtype=np.int64)
        rc = self.lib.oracle_tiled_matmul_count(self._p(A), self._p(Bm), self._p(out),
                                                M, N, K, bm, bn, bk, self._p(counts))
        if rc:
            raise ValueError("oracle_tiled_matmul_count rejected its arguments")
        return out, int(counts[0]), int(counts[1]), int(counts[2]), int(counts[3])


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``oracle/oracle.c`` (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
