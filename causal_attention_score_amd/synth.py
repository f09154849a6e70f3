"""Seeded synthetic inputs shared by the HIP path's tests, the benchmark and the
oracle's tests.

This module holds no arithmetic of the method itself: it only draws numbers
(numpy ``default_rng``, the PCG64 bit generator), rounds them to the storage
type (fp32, or round-to-nearest-even bfloat16 / binary16) and lays them out in
the shapes the pages use. The same bits go to the GPU and to the oracle.

Workloads (sizes from the pages):
  * dense fp32 15x9x12, uniform[0,1) -- the kernl "1 - tiled matmul" notebook.
  * dense fp32 X[960,770] . W[1024,770]^T, N(0,1)/sqrt(770) -- the DietCode
    local-padding dense layer (B=16, T=60, I=770) with H=1024.
  * causal scores fp32, QKV (8,1024,3,12,64), N(0,1) -- the llm.c
    trimat_forward.cu benchmark shape.
  * dense bf16 4096^3, N(0,1).
  * causal scores bf16, QKV (4,4096,3,25,64), N(0,1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def uniform01_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.random(size=shape, dtype=np.float64).astype(np.float32)


def normal_f32(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float64)
    if scale != 1.0:
        x = x * scale
    return x.astype(np.float32)


def small_int_f32(g: np.random.Generator, shape, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Integers in [lo, hi]: exact in every storage type, and every partial sum
    of their products is an integer, so any summation order gives one result."""
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to IEEE binary16 (numpy's cast is nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_storage(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage array: float32 for f32, uint16 bits otherwise."""
    if dtype == "f32":
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x_f32)
    if dtype == "f16":
        return f16_bits(x_f32)
    raise ValueError(dtype)


# ------------------------------------------------------------------ inputs

def gemm_inputs(M: int, N: int, K: int, dtype: str = "f32", seed: int = 0,
                dist: str = "normal", scale: float = 1.0):
    """X [M, K] then W [N, K], drawn in that order from one generator."""
    g = rng(seed)
    draw = {"normal": lambda s: normal_f32(g, s, scale),
            "uniform": lambda s: uniform01_f32(g, s),
            "int": lambda s: small_int_f32(g, s)}[dist]
    X = draw((M, K))
    W = draw((N, K))
    return to_storage(X, dtype), to_storage(W, dtype)


def trimul_inputs(B: int, T: int, NH: int, HS: int, dtype: str = "f32", seed: int = 0,
                  dist: str = "normal"):
    """Packed QKV laid out (B, T, 3, NH, HS), returned flat as [B, T, 3*NH*HS]."""
    g = rng(seed)
    shape = (B, T, 3 * NH * HS)
    if dist == "normal":
        x = normal_f32(g, shape)
    elif dist == "int":
        x = small_int_f32(g, shape)
    else:
        x = uniform01_f32(g, shape)
    return to_storage(x, dtype)


def ramp_qk_inputs(B: int, T: int, NH: int, HS: int, q0, dtype: str = "f32", v_ramp: bool = False,
                   v_seed: int | None = None):
    """Structured packed QKV: head entry 0 of Q is q0[nh] on every row, entry
    0 of K is the row index t2, every other Q and K entry is zero. The dot
    product of Q row t and K row t2 in head nh is then q0[nh] * t2, the same
    ramp on every row, one product (exact in fp32 when it fits 24 bits). V is
    zero, or N(0,1) drawn from v_seed; with v_ramp its entry 0 is the row
    index. Q and K values should be exact in the storage type (a rounded key
    index still gives one exact product, only not a ramp)."""
    x = np.zeros((B, T, 3, NH, HS), dtype=np.float32)
    x[:, :, 0, :, 0] = np.asarray(q0, dtype=np.float32)[None, None, :]
    x[:, :, 1, :, 0] = np.arange(T, dtype=np.float32)[None, :, None]
    if v_seed is not None:
        x[:, :, 2] = normal_f32(rng(v_seed), (B, T, NH, HS))
    if v_ramp:
        x[:, :, 2, :, 0] = np.arange(T, dtype=np.float32)[None, :, None]
    return to_storage(x.reshape(B, T, 3 * NH * HS), dtype)


# --------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "gemm_nt", "batch_matmul_nt" or "trimul_causal"
    dtype: str           # input storage type; outputs are fp32
    seed: int
    dims: tuple          # gemm: (M, N, K); batched: (batch, M, N, K); trimul: (B, T, NH, HS)
    dist: str = "normal"
    scale: float = 1.0   # multiplier applied in double before rounding

    def inputs(self):
        if self.kind == "gemm_nt":
            M, N, K = self.dims
            if self.dist == "uniform":
                # A [M, K] then B [K, N] as drawn by the notebook; the NT entry
                # point takes W = B^T, an exact host-side transpose.
                g = rng(self.seed)
                A = uniform01_f32(g, (M, K))
                Bm = uniform01_f32(g, (K, N))
                return to_storage(A, self.dtype), to_storage(np.ascontiguousarray(Bm.T), self.dtype)
            return gemm_inputs(M, N, K, self.dtype, self.seed, self.dist, self.scale)
        if self.kind == "batch_matmul_nt":
            Bt, M, N, K = self.dims
            X, W = gemm_inputs(Bt * M, Bt * N, K, self.dtype, self.seed, self.dist, self.scale)
            return X.reshape(Bt, M, K), W.reshape(Bt, N, K)
        B, T, NH, HS = self.dims
        return (trimul_inputs(B, T, NH, HS, self.dtype, self.seed, self.dist),)

    def useful_flops(self) -> int:
        if self.kind == "gemm_nt":
            M, N, K = self.dims
            return 2 * M * N * K
        if self.kind == "batch_matmul_nt":
            Bt, M, N, K = self.dims
            return 2 * Bt * M * N * K
        B, T, NH, HS = self.dims
        return 2 * HS * B * NH * T * (T + 1) // 2

    def algorithmic_bytes(self, out_bytes: int = 4) -> int:
        """Each operand read once and the full output written once (for the
        scores: Q and K read, V never read, the whole (T, T) plane written in
        elements of out_bytes)."""
        es = 4 if self.dtype == "f32" else 2
        if self.kind == "gemm_nt":
            M, N, K = self.dims
            return es * (M * K + N * K) + 4 * M * N
        if self.kind == "batch_matmul_nt":
            Bt, M, N, K = self.dims
            return Bt * (es * (M * K + N * K) + 4 * M * N)
        B, T, NH, HS = self.dims
        return es * 2 * B * T * NH * HS + out_bytes * B * NH * T * T


WORKLOADS = {
    "dense_f32_15x9x12": Workload("dense_f32_15x9x12", "gemm_nt", "f32", 1, (15, 9, 12), "uniform"),
    "dense_f32_960x1024x770": Workload("dense_f32_960x1024x770", "gemm_nt", "f32", 2,
                                       (960, 1024, 770), "normal", 1.0 / np.sqrt(770.0)),
    "trimul_f32_B8_T1024_NH12_HS64": Workload("trimul_f32_B8_T1024_NH12_HS64", "trimul_causal",
                                              "f32", 3, (8, 1024, 12, 64)),
    "dense_bf16_4096": Workload("dense_bf16_4096", "gemm_nt", "bf16", 4, (4096, 4096, 4096)),
    # The local-padding A/B shape of DietCode's test_local_padding (B=16,
    # T=60, I=770, H=2304): the same inputs recipe as the 1024-wide layer.
    "dense_f32_960x2304x770": Workload("dense_f32_960x2304x770", "gemm_nt", "f32", 6,
                                       (960, 2304, 770), "normal", 1.0 / np.sqrt(770.0)),
    # BatchMatmulNT of DietCode's test_local_padding_ii (B=16, T=120, H=768,
    # NH=12: B*NH = 192 heads of 120 x 120 x 64), and the causal scores of the
    # same heads read from packed QKV (ragged T: 120 is not a tile multiple).
    "bmm_nt_f32_192x120x120x64": Workload("bmm_nt_f32_192x120x120x64", "batch_matmul_nt", "f32", 7,
                                          (192, 120, 120, 64)),
    "trimul_f32_B16_T120_NH12_HS64": Workload("trimul_f32_B16_T120_NH12_HS64", "trimul_causal", "f32", 8,
                                              (16, 120, 12, 64)),
    # binary16 inputs at the two large shapes (the scores are also timed with
    # 16-bit outputs).
    "dense_f16_4096": Workload("dense_f16_4096", "gemm_nt", "f16", 9, (4096, 4096, 4096)),
    "trimul_f16_B4_T4096_NH25_HS64": Workload("trimul_f16_B4_T4096_NH25_HS64", "trimul_causal", "f16", 10,
                                              (4, 4096, 25, 64)),
    "trimul_bf16_B4_T4096_NH25_HS64": Workload("trimul_bf16_B4_T4096_NH25_HS64", "trimul_causal",
                                               "bf16", 5, (4, 4096, 25, 64)),
}
