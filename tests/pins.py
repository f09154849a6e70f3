"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes a loaded oracle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with:
  * exact rational arithmetic on tiny inputs (Python ``fractions``), with the
    operands sliced out of the packed layout by numpy reshapes, an indexing
    route independent of the oracle's pointer arithmetic;
  * the closed form of the ramp inputs of the tensor-core study blog
    ("Tensor Core学习", the sgemm_wmma_naive test main: A = i/256 and
    B = (i+1.25)/128 read as an NT pair);
  * the worked tiling example of the kernl notebook "1 - tiled matmul"
    (864 loads, 135 writes, stored in tests/golden/);
  * identity, zero and empty products, and the closed forms of the tile
    counts on ragged shapes;
  * invariants of the causal scores (lower triangle = scaled dense product,
    NaN count, non-negative diagonal when Q = K) and thread-count
    independence;
  * library conversions of bfloat16 / binary16 (torch, numpy);
  * for the causal softmax: the closed form of geometric score rows, the
    max-free formula 1 / sum exp(s_k - s) on exact scores, rows summing to
    one, saturated rows, and the pinned score oracle's row maxima;
  * for the attention output: row 0 equals V's row 0, all-ones V gives ones,
    uniform scores give running means, ramp scores give the expectation of
    a truncated geometric law, and a max-free formula on exact scores.

The same functions run against mutated copies of the oracle in
test_oracle_mutations.py, which checks that every planted mistake is caught.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from causal_attention_score_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
QNAN = 0x7FC00000


# ------------------------------------------------------------------ helpers

def f32_round(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # choose e so that 2^23 <= a / 2^(e-23) < 2^24
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 23, -149)  # quantum; subnormals keep the fixed -149 quantum
    n = round(a / Fraction(2) ** q)  # Fraction.__round__ is ties-to-even
    return np.float32(sign * n * 2.0 ** q)


def ulp32(x: float) -> float:
    x = np.float32(abs(x))
    return float(np.nextafter(x, np.float32(np.inf)) - x) if x != 0 else 2.0 ** -149


def bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def decoded(orc, a, dtype):
    return orc.decode(a, dtype) if dtype != "f32" else np.asarray(a, dtype=np.float64)


def exact_gemm(X, W, dtype, orc):
    """Exact rational Y = X W^T and sum |x w|, operands widened by the library
    conversions (numpy for fp32/f16, torch for bf16), not by the oracle."""
    Xd, Wd = lib_decode(X, dtype), lib_decode(W, dtype)
    M, K = Xd.shape
    N = Wd.shape[0]
    Y = [[None] * N for _ in range(M)]
    S = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            asum = Fraction(0)
            for k in range(K):
                p = Fraction(float(Xd[m, k])) * Fraction(float(Wd[n, k]))
                acc += p
                asum += abs(p)
            Y[m][n], S[m][n] = acc, asum
    return Y, S


def lib_decode(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    import torch
    t = torch.from_numpy(a.astype(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def scale_is_nearest(s: np.float32, hs: int) -> bool:
    """s is the binary32 value nearest to 1/sqrt(hs): 1/hs lies between the
    squares of the midpoints to s's neighbours (exact rationals)."""
    lo = np.nextafter(s, np.float32(0))
    hi = np.nextafter(s, np.float32(np.inf))
    fs, flo, fhi = Fraction(float(s)), Fraction(float(lo)), Fraction(float(hi))
    target = Fraction(1, hs)
    return ((flo + fs) / 2) ** 2 <= target <= ((fs + fhi) / 2) ** 2


# ------------------------------------------------------------- gemm pins

def pin_gemm_bruteforce_int(orc):
    for (M, N, K, seed) in [(1, 1, 1, 0), (3, 5, 7, 1), (8, 8, 8, 2), (5, 2, 6, 3)]:
        for dtype in ("f32", "bf16", "f16"):
            X, W = synth.gemm_inputs(M, N, K, dtype, seed, dist="int")
            Y, bound = orc.gemm_nt(X, W, dtype)
            Ye, Se = exact_gemm(X, W, dtype, orc)
            for m in range(M):
                for n in range(N):
                    assert bits(Y[m, n]) == bits(f32_round(Ye[m][n])), (dtype, M, N, K, m, n)
                    assert Fraction(float(bound[m, n])) == Se[m][n], (dtype, m, n)


def pin_gemm_bruteforce_random(orc):
    for (M, N, K, seed) in [(4, 3, 5, 10), (7, 6, 8, 11)]:
        for dtype in ("f32", "bf16"):
            X, W = synth.gemm_inputs(M, N, K, dtype, seed, dist="normal")
            Y, bound = orc.gemm_nt(X, W, dtype)
            Ye, Se = exact_gemm(X, W, dtype, orc)
            for m in range(M):
                for n in range(N):
                    ref = f32_round(Ye[m][n])
                    # one rounding of the exact sum; a double-sum error can tip
                    # a near-tie by at most one unit in the last place
                    assert abs(float(Y[m, n]) - float(ref)) <= ulp32(float(ref)), (dtype, m, n)
                    assert abs(Fraction(float(bound[m, n])) - Se[m][n]) <= Se[m][n] * Fraction(1, 2 ** 48)


def pin_batch_matmul_bruteforce(orc):
    """Every block of the batched product is its own exact dense product
    (a wrong batch index for X or W, or a transposed block, fails)."""
    for dtype in ("f32", "bf16"):
        Bt, M, N, K = 3, 2, 3, 5
        X, W = synth.gemm_inputs(Bt * M, Bt * N, K, dtype, 21, dist="int")
        X, W = X.reshape(Bt, M, K), W.reshape(Bt, N, K)
        Y, bound = orc.batch_matmul_nt(X, W, dtype)
        for i in range(Bt):
            Ye, Se = exact_gemm(X[i], W[i], dtype, orc)
            for m in range(M):
                for n in range(N):
                    assert bits(Y[i, m, n]) == bits(f32_round(Ye[m][n])), (dtype, i, m, n)
                    assert Fraction(float(bound[i, m, n])) == Se[m][n], (dtype, i, m, n)


def pin_round16_against_libraries(orc):
    """16-bit storage rounding against numpy's binary16 conversion and
    torch's bfloat16 conversion (both round to nearest even), over random
    values of every magnitude, every binary16 tie, and the edges."""
    import torch
    g = np.random.default_rng(5)
    mags = np.exp2(g.uniform(-30, 20, 200000)).astype(np.float32)
    vals = mags * np.where(g.random(mags.size) < 0.5, -1, 1).astype(np.float32)
    bits32 = g.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    rand_bits = bits32.view(np.float32)
    rand_bits = rand_bits[~np.isnan(rand_bits)]
    # binary16 ties: halfway between neighbours (exact in binary32)
    h = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    hn = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    ties = ((h + hn) / 2).astype(np.float32)
    edges = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30, -1e30, np.inf, -np.inf,
                      2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
                      3.3895314e38, 3.4028235e38, 1.1754944e-38, 1e-45], dtype=np.float32)
    for x in (vals, rand_bits, ties, edges):
        f16 = orc.round16(x, "f16")
        with np.errstate(over="ignore"):  # values past the binary16 range become infinity
            ref16 = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(f16, ref16), "binary16 rounding"
        b16 = orc.round16(x, "bf16")
        ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(b16, ref), "bfloat16 rounding"
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(orc.round16(nan, "bf16") == 0x7FC0) and np.all(orc.round16(nan, "f16") == 0x7E00)


def pin_round16_worked_values(orc):
    """Hand-derived cases: binary16 keeps 11 significant bits, so 1 + 2^-11
    is a tie between 1 and 1 + 2^-10 and goes to the even 1, while
    1 + 3*2^-11, a tie between 1 + 2^-10 and 1 + 2^-9, goes to the even
    1 + 2^-9; bfloat16 keeps 8 significant bits (ties at 2^-8 likewise)."""
    cases16 = [(1.0 + 2.0 ** -11, 0x3C00),           # tie below: even 1.0
               (1.0 + 3 * 2.0 ** -11, 0x3C02),       # tie between 0x3C01 and 0x3C02: even 0x3C02
               (65519.0, 0x7BFF), (65520.0, 0x7C00),  # the overflow midpoint goes to infinity
               (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002), (2.0 ** -24, 0x0001)]
    for v, b in cases16:
        assert int(orc.round16(np.array([v], np.float32), "f16")[0]) == b, (v, hex(b))
    cases_bf = [(1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82), (-2.0, 0xC000),
                (3.3961775e38, 0x7F80)]                 # above the largest finite bfloat16: infinity
    for v, b in cases_bf:
        assert int(orc.round16(np.array([v], np.float32), "bf16")[0]) == b, (v, hex(b))


def pin_gemm_strided(orc):
    """Row pitches larger than K: only the first K entries of a row count."""
    M, N, K, ldx, ldw, ldy = 5, 4, 3, 7, 6, 9
    g = np.random.default_rng(5)
    Xf = g.integers(-3, 4, size=(M, ldx)).astype(np.float32)
    Wf = g.integers(-3, 4, size=(N, ldw)).astype(np.float32)
    Y, _ = orc.gemm_nt(Xf, Wf, "f32", M=M, N=N, K=K, ldx=ldx, ldw=ldw, ldy=ldy)
    ref = Xf[:, :K].astype(np.int64) @ Wf[:, :K].astype(np.int64).T
    assert np.array_equal(Y[:, :N], ref.astype(np.float32))
    assert np.all(Y[:, N:] == 0)  # columns past N are never written


def pin_gemm_ramp_closed_form(orc):
    """Ramp inputs of the tensor-core blog's WMMA test, read as NT:
    A[m,k] = (mK+k)/256, W[n,k] = (nK+k+1.25)/128. With a = mK and
    c = nK + 1.25, Y = (K a c + (a+c) K(K-1)/2 + (K-1)K(2K-1)/6) / 32768."""
    for (M, N, K) in [(16, 16, 16), (5, 7, 13), (1, 3, 64)]:
        A = (np.arange(M * K, dtype=np.float64) / 256.0).astype(np.float32).reshape(M, K)
        W = ((np.arange(N * K, dtype=np.float64) + 1.25) / 128.0).astype(np.float32).reshape(N, K)
        Y, _ = orc.gemm_nt(A, W, "f32")
        for m in range(M):
            for n in range(N):
                a = Fraction(m * K)
                c = Fraction(n * K) + Fraction(5, 4)
                exact = (K * a * c + (a + c) * Fraction(K * (K - 1), 2)
                         + Fraction((K - 1) * K * (2 * K - 1), 6)) / 32768
                assert bits(Y[m, n]) == bits(f32_round(exact)), (M, N, K, m, n)


def pin_gemm_identity_zero_empty(orc):
    g = np.random.default_rng(7)
    X = g.standard_normal((6, 9)).astype(np.float32)
    Y, _ = orc.gemm_nt(X, np.eye(9, dtype=np.float32), "f32")
    assert np.array_equal(bits(Y), bits(X))
    Y, _ = orc.gemm_nt(np.eye(6, dtype=np.float32), X.T.copy(), "f32")  # I . (X^T)^T = X
    assert np.array_equal(bits(Y), bits(X))
    Y, _ = orc.gemm_nt(np.zeros((4, 5), np.float32), g.standard_normal((3, 5)).astype(np.float32), "f32")
    assert np.all(Y == 0)
    Y, b = orc.gemm_nt(np.zeros((4, 0), np.float32), np.zeros((3, 0), np.float32), "f32")
    assert Y.shape == (4, 3) and np.all(Y == 0) and np.all(b == 0)  # empty sum


# ------------------------------------------------------------ trimul pins

def qk_views(qkv, B, T, NH, HS, dtype):
    """Q and K as (B, NH, T, HS) via numpy reshape of the packed
    (B, T, 3, NH, HS) layout, decoded by the library conversions."""
    d = lib_decode(qkv, dtype).reshape(B, T, 3, NH, HS)
    return d[:, :, 0].transpose(0, 2, 1, 3), d[:, :, 1].transpose(0, 2, 1, 3)


def pin_trimul_scale(orc):
    for hs in (1, 2, 3, 5, 8, 40, 64, 80, 96, 128, 255):
        s = orc.trimul_scale(hs)
        assert scale_is_nearest(s, hs), hs
    assert orc.trimul_scale(64) == np.float32(0.125)


def pin_trimul_bruteforce(orc):
    for (B, T, NH, HS, seed, dist, dtype) in [
        (1, 1, 1, 1, 0, "int", "f32"),
        (2, 9, 2, 5, 1, "int", "f32"),
        (1, 7, 3, 4, 2, "int", "bf16"),
        (2, 5, 2, 3, 3, "normal", "f32"),
        (1, 6, 2, 8, 4, "normal", "f16"),
    ]:
        C = NH * HS
        qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed, dist)
        out, bound = orc.trimul_causal(qkv, B, T, C, NH, dtype)
        Q, Kt = qk_views(qkv, B, T, NH, HS, dtype)
        s = Fraction(float(orc.trimul_scale(HS)))
        for b in range(B):
            for h in range(NH):
                for t in range(T):
                    for t2 in range(T):
                        v = out[b, h, t, t2]
                        if t2 > t:
                            assert bits(v) == QNAN, (b, h, t, t2)
                            continue
                        dot = sum((Fraction(float(Q[b, h, t, i])) * Fraction(float(Kt[b, h, t2, i]))
                                   for i in range(HS)), Fraction(0))
                        asum = sum((abs(Fraction(float(Q[b, h, t, i])) * Fraction(float(Kt[b, h, t2, i])))
                                    for i in range(HS)), Fraction(0))
                        ref = f32_round(dot * s)
                        tol = 0 if dist == "int" else ulp32(float(ref))
                        assert abs(float(v) - float(ref)) <= tol, (dtype, b, h, t, t2, v, ref)
                        assert abs(Fraction(float(bound[b, h, t, t2])) - asum * s) <= asum * s * Fraction(1, 2 ** 48)


def pin_trimul_vs_numpy_matmul(orc):
    """Lower triangle equals scale * (Q @ K^T) from numpy's float64 matmul."""
    B, T, NH, HS = 2, 37, 3, 16
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", 21)
    out, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32")
    Q, Kt = qk_views(qkv, B, T, NH, HS, "f32")
    ref = (Q @ Kt.transpose(0, 1, 3, 2)) * float(orc.trimul_scale(HS))
    low = np.tril(np.ones((T, T), dtype=bool))
    err = np.abs(out.astype(np.float64) - ref)[..., low]
    assert np.all(err <= 1e-6 * bound[..., low] + 1e-30), err.max()
    assert np.all(bits(out[..., ~low]) == QNAN)


def pin_trimul_equals_dense_lower(orc):
    """trimul = scale * lower(gemm_nt(Q, K)) per (b, nh); with HS = 64 the
    scale is 1/8, a power of two, so the two agree bit for bit."""
    B, T, NH, HS = 2, 19, 2, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", 22)
    out, _ = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32")
    d = qkv.reshape(B, T, 3, NH, HS)
    low = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(NH):
            Y, _ = orc.gemm_nt(np.ascontiguousarray(d[b, :, 0, h]), np.ascontiguousarray(d[b, :, 1, h]), "f32")
            assert np.array_equal(bits(out[b, h][low]), bits((Y * np.float32(0.125))[low]))


def pin_trimul_mask_counts(orc):
    for (B, T, NH, HS) in [(1, 1, 1, 4), (2, 13, 3, 4), (1, 64, 2, 8)]:
        qkv = synth.trimul_inputs(B, T, NH, HS, "f32", 23)
        out, _ = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32")
        u = bits(out)
        assert int(np.sum(u == QNAN)) == B * NH * T * (T - 1) // 2
        assert int(np.sum(np.isfinite(out))) == B * NH * T * (T + 1) // 2


def pin_trimul_q_equals_k(orc):
    """With K = Q the diagonal is scale * |q_t|^2 >= 0 and the lower triangle
    is symmetric with the transposed product."""
    B, T, NH, HS = 1, 11, 2, 6
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", 24).reshape(B, T, 3, NH, HS)
    qkv[:, :, 1] = qkv[:, :, 0]
    out, _ = orc.trimul_causal(qkv.reshape(B, T, -1), B, T, NH * HS, NH, "f32")
    Q = qkv[0, :, 0].astype(np.float64)          # (T, NH, HS)
    s = float(orc.trimul_scale(HS))
    for h in range(NH):
        diag = np.diagonal(out[0, h])
        assert np.all(diag >= 0)
        ref = s * np.sum(Q[:, h] ** 2, axis=1)
        assert np.allclose(diag, ref, rtol=1e-6, atol=0)


def pin_trimul_rows_match_full(orc):
    B, T, NH, HS = 2, 21, 3, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", 25)
    full, _ = orc.trimul_causal(qkv, B, T, NH * HS, NH, "bf16")
    part, _ = orc.trimul_causal_rows(qkv, B, T, NH * HS, NH, 1, 2, 5, 17, "bf16")
    assert np.array_equal(bits(part), bits(full[1, 2, 5:17]))


def pin_thread_independence(orc):
    n0 = orc.num_threads()
    try:
        X, W = synth.gemm_inputs(67, 45, 129, "f32", 26)
        qkv = synth.trimul_inputs(2, 70, 2, 24, "bf16", 27)
        orc.set_threads(1)
        y1, _ = orc.gemm_nt(X, W, "f32")
        o1, _ = orc.trimul_causal(qkv, 2, 70, 48, 2, "bf16")
        orc.set_threads(max(2, os.cpu_count() or 2))
        y2, _ = orc.gemm_nt(X, W, "f32")
        o2, _ = orc.trimul_causal(qkv, 2, 70, 48, 2, "bf16")
        assert np.array_equal(bits(y1), bits(y2)) and np.array_equal(bits(o1), bits(o2))
    finally:
        orc.set_threads(n0)


# ------------------------------------------------------------ softmax pins

def geometric_row(slope: float, t: int):
    """Closed form of the softmax of the row (slope * k for k = 0..t):
    returns (max, ln sum exp(x - max)). The shifted terms are the geometric
    series e^(-|slope| j), j = 0..t, whose sum is (1 - r^(t+1)) / (1 - r)."""
    n = t + 1
    if slope == 0:
        return 0.0, math.log(n)
    a = abs(slope)
    mx = slope * t if slope > 0 else 0.0
    return mx, math.log(-math.expm1(-a * n)) - math.log(-math.expm1(-a))


def pin_softmax_geometric_closed_form(orc):
    """Score rows that are exact ramps slope * t2 (HS = 64, scale = 1/8):
    row max, log-sum, every log-probability and probability against the
    closed form of a truncated geometric series."""
    B, T, NH, HS = 2, 40, 3, 64
    slopes = [0.25, -0.5, 0.0]
    for dtype in ("f32", "bf16", "f16"):
        qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in slopes], dtype)
        C = NH * HS
        lp, mx, ls, _ = orc.causal_softmax(qkv, B, T, C, NH, dtype, "log", with_bound=False)
        pr, mx2, ls2, _ = orc.causal_softmax(qkv, B, T, C, NH, dtype, "prob", with_bound=False)
        assert np.array_equal(mx, mx2) and np.array_equal(ls, ls2)
        for b in range(B):
            for h, a in enumerate(slopes):
                for t in range(T):
                    m_ref, l_ref = geometric_row(a, t)
                    assert abs(mx[b, h, t] - m_ref) <= 1e-13, (dtype, h, t, mx[b, h, t], m_ref)
                    assert abs(ls[b, h, t] - l_ref) <= 1e-13, (dtype, h, t, ls[b, h, t], l_ref)
                    ref = np.array([a * k - m_ref - l_ref for k in range(t + 1)])
                    assert np.max(np.abs(lp[b, h, t, :t + 1] - ref)) <= 1e-12, (dtype, h, t)
                    assert np.max(np.abs(pr[b, h, t, :t + 1] - np.exp(ref))) <= 1e-13, (dtype, h, t)


def pin_softmax_maxfree_formula(orc):
    """Small-integer inputs, exact rational scores: every probability equals
    1 / sum_k exp(s_k - s_t2) (no maximum, no logarithm of the sum), evaluated
    with math.fsum, and the row maximum is the largest exact score."""
    for (B, T, NH, HS, seed, dtype) in [(2, 6, 2, 4, 31, "f32"), (1, 7, 3, 8, 32, "bf16"), (1, 5, 2, 3, 33, "f16")]:
        C = NH * HS
        qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed, "int")
        pr, mx, ls, _ = orc.causal_softmax(qkv, B, T, C, NH, dtype, "prob", with_bound=False)
        lp, _, _, _ = orc.causal_softmax(qkv, B, T, C, NH, dtype, "log", with_bound=False)
        Q, Kt = qk_views(qkv, B, T, NH, HS, dtype)
        sc = Fraction(float(orc.trimul_scale(HS)))
        for b in range(B):
            for h in range(NH):
                for t in range(T):
                    s = [float(sc * sum((Fraction(float(Q[b, h, t, i])) * Fraction(float(Kt[b, h, k, i]))
                                         for i in range(HS)), Fraction(0))) for k in range(t + 1)]
                    assert mx[b, h, t] == max(s), (dtype, b, h, t)
                    for t2 in range(T):
                        if t2 > t:
                            assert pr[b, h, t, t2] == 0.0 and lp[b, h, t, t2] == -np.inf
                            continue
                        z = math.fsum(math.exp(sk - s[t2]) for sk in s)
                        assert abs(pr[b, h, t, t2] - 1.0 / z) <= 1e-14 * (1.0 / z) + 1e-300, (dtype, b, h, t, t2)
                        assert abs(lp[b, h, t, t2] + math.log(z)) <= 1e-13, (dtype, b, h, t, t2)


def pin_softmax_rows_sum_to_one(orc):
    """Every causal row of probabilities sums to one; masked entries are
    exactly 0 (probabilities) and -inf (log-probabilities); exp of the
    log-probabilities gives the probabilities; the largest log-probability of
    a row is -logsum, and 0 <= logsum <= ln(t + 1)."""
    B, T, NH, HS = 2, 33, 2, 16
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", 34)
    pr, mx, ls, _ = orc.causal_softmax(qkv, B, T, NH * HS, NH, "f32", "prob", with_bound=False)
    lp, _, _, _ = orc.causal_softmax(qkv, B, T, NH * HS, NH, "f32", "log", with_bound=False)
    up = np.triu(np.ones((T, T), dtype=bool), 1)
    assert np.all(pr[..., up] == 0.0) and np.all(lp[..., up] == -np.inf)
    assert np.all(np.isfinite(lp[..., ~up]))
    for b in range(B):
        for h in range(NH):
            for t in range(T):
                assert abs(math.fsum(pr[b, h, t]) - 1.0) <= 1e-13, (b, h, t)
                assert abs(np.max(lp[b, h, t]) + ls[b, h, t]) <= 1e-15
                assert -1e-15 <= ls[b, h, t] <= math.log(t + 1) + 1e-13
    low = ~up
    assert np.allclose(np.exp(lp[..., low]), pr[..., low], rtol=1e-13, atol=0)


def pin_softmax_saturated(orc):
    """Scores of order 1e3-1e4 (exp of a raw score overflows double): the
    outputs stay finite, rows sum to one, and the row maximum is the largest
    score of the pinned score oracle up to its fp32 rounding."""
    B, T, NH, HS = 1, 24, 2, 16
    qkv = (synth.trimul_inputs(B, T, NH, HS, "f32", 35) * np.float32(64.0)).astype(np.float32)
    pr, mx, ls, _ = orc.causal_softmax(qkv, B, T, NH * HS, NH, "f32", "prob", with_bound=False)
    sc, _ = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32", with_bound=False)
    assert np.max(np.abs(mx)) > 800.0
    assert np.all(np.isfinite(ls))
    for b in range(B):
        for h in range(NH):
            for t in range(T):
                assert abs(math.fsum(pr[b, h, t]) - 1.0) <= 1e-13
                smax = float(np.max(sc[b, h, t, :t + 1]))
                assert abs(mx[b, h, t] - smax) <= ulp32(smax), (b, h, t, mx[b, h, t], smax)


def pin_softmax_rows_match_full(orc):
    B, T, NH, HS = 2, 21, 3, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, "f16", 36)
    for mode in ("log", "prob"):
        full, mx, ls, bd = orc.causal_softmax(qkv, B, T, NH * HS, NH, "f16", mode)
        part, pmx, pls, pbd = orc.causal_softmax_rows(qkv, B, T, NH * HS, NH, 1, 2, 5, 17, "f16", mode)
        assert np.array_equal(part, full[1, 2, 5:17]) and np.array_equal(pbd, bd[1, 2, 5:17])
        assert np.array_equal(pmx, mx[1, 2, 5:17]) and np.array_equal(pls, ls[1, 2, 5:17])
    _, tb = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f16")
    assert np.array_equal(bd, tb)  # the same error scale as the scores


# ---------------------------------------------------- attention-output pins

def v_views(qkv, B, T, NH, HS, dtype):
    """V as (B, NH, T, HS), sliced from the packed layout by numpy reshapes."""
    d = lib_decode(qkv, dtype).reshape(B, T, 3, NH, HS)
    return d[:, :, 2].transpose(0, 2, 1, 3)


def pin_attention_first_row_and_ones(orc):
    """Row 0 attends only to itself (p = 1): y equals V's row 0 exactly. With
    V all ones, every output is 1 (the probabilities sum to one)."""
    B, T, NH, HS = 2, 17, 3, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", 41)
    y, _ = orc.causal_attention(qkv, B, T, NH * HS, NH, "f32")
    V = v_views(qkv, B, T, NH, HS, "f32")
    assert np.array_equal(y[:, 0, :].reshape(B, NH, HS), V[:, :, 0, :])
    ones = qkv.reshape(B, T, 3, NH * HS).copy()
    ones[:, :, 2] = 1.0
    y1, _ = orc.causal_attention(ones.reshape(B, T, -1), B, T, NH * HS, NH, "f32")
    assert np.max(np.abs(y1 - 1.0)) <= 1e-13


def pin_attention_uniform_is_running_mean(orc):
    """Q = 0 makes every score 0, so p = 1/(t+1) and y[t] is the mean of V's
    rows 0..t (numpy cumulative sums)."""
    B, T, NH, HS = 1, 30, 2, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", 42)
    d = qkv.reshape(B, T, 3, NH * HS).copy()
    d[:, :, 0] = 0
    d = d.reshape(B, T, -1)
    y, _ = orc.causal_attention(d, B, T, NH * HS, NH, "bf16")
    V = lib_decode(d, "bf16").reshape(B, T, 3, NH * HS)[:, :, 2]
    mean = np.cumsum(V, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert np.max(np.abs(y - mean)) <= 1e-12


def pin_attention_ramp_expectation(orc):
    """Ramp scores a * t2 with V entry 0 = t2: y[t][0] is the expectation of
    k under p_k proportional to exp(a k), k = 0..t (direct sums with
    math.fsum, no maximum taken); the other entries are 0."""
    B, T, NH, HS = 1, 40, 3, 64
    slopes = [0.25, -0.5, 0.0]
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in slopes], "f32", v_ramp=True)
    y, _ = orc.causal_attention(qkv, B, T, NH * HS, NH, "f32")
    y = y.reshape(B, T, NH, HS)
    for h, a in enumerate(slopes):
        for t in range(T):
            w = [math.exp(a * k) for k in range(t + 1)]
            ref = math.fsum(k * wk for k, wk in enumerate(w)) / math.fsum(w)
            assert abs(y[0, t, h, 0] - ref) <= 1e-12 * max(1.0, ref), (h, t, y[0, t, h, 0], ref)
            assert np.all(y[0, t, h, 1:] == 0.0)


def pin_attention_maxfree_bruteforce(orc):
    """Small-integer inputs, exact rational scores: y_t = sum_j v_j / sum_k
    exp(s_k - s_j) (no maximum, no logarithm), via math.fsum."""
    for (B, T, NH, HS, seed, dtype) in [(2, 6, 2, 4, 43, "f32"), (1, 5, 2, 8, 44, "f16")]:
        C = NH * HS
        qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed, "int")
        y, aw = orc.causal_attention(qkv, B, T, C, NH, dtype)
        Q, Kt = qk_views(qkv, B, T, NH, HS, dtype)
        V = v_views(qkv, B, T, NH, HS, dtype)
        sc = Fraction(float(orc.trimul_scale(HS)))
        for b in range(B):
            for h in range(NH):
                for t in range(T):
                    s = [float(sc * sum((Fraction(float(Q[b, h, t, i])) * Fraction(float(Kt[b, h, k, i]))
                                         for i in range(HS)), Fraction(0))) for k in range(t + 1)]
                    p = [1.0 / math.fsum(math.exp(sk - sj) for sk in s) for sj in s]
                    for i in range(HS):
                        ref = math.fsum(p[j] * float(V[b, h, j, i]) for j in range(t + 1))
                        aref = math.fsum(p[j] * abs(float(V[b, h, j, i])) for j in range(t + 1))
                        assert abs(y[b, t, h * HS + i] - ref) <= 1e-13 * max(1.0, aref), (dtype, b, h, t, i)
                        assert abs(aw[b, t, h * HS + i] - aref) <= 1e-13 * max(1.0, aref)


def pin_attention_saturated(orc):
    """Scores of order 1e3-1e4 with V all ones: every output is 1 and finite
    (exp of an unshifted score overflows; the row maximum keeps it in range)."""
    B, T, NH, HS = 1, 24, 2, 16
    qkv = (synth.trimul_inputs(B, T, NH, HS, "f32", 46) * np.float32(64.0)).astype(np.float32)
    d = qkv.reshape(B, T, 3, NH * HS).copy()
    d[:, :, 2] = 1.0
    y, aw = orc.causal_attention(d.reshape(B, T, -1), B, T, NH * HS, NH, "f32")
    assert np.all(np.isfinite(y)) and np.max(np.abs(y - 1.0)) <= 1e-12
    assert np.max(np.abs(aw - 1.0)) <= 1e-12


def pin_attention_rows_match_full(orc):
    B, T, NH, HS = 2, 21, 3, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", 45)
    full, fa = orc.causal_attention(qkv, B, T, NH * HS, NH, "bf16")
    part, pa = orc.causal_attention(qkv, B, T, NH * HS, NH, "bf16", b_range=[1], t_range=(5, 17))
    assert np.array_equal(part[0], full[1, 5:17]) and np.array_equal(pa[0], fa[1, 5:17])


# ------------------------------------------------------- tiled-count pins

def read_golden_counts():
    vals = {}
    with open(os.path.join(GOLDEN, "kernl_tiled_matmul_counts.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals


def pin_tiled_worked_example(orc):
    g = read_golden_counts()
    M, N, K = g["M"], g["N"], g["K"]
    wl = synth.WORKLOADS["dense_f32_15x9x12"]
    A, Wt = wl.inputs()
    Bm = np.ascontiguousarray(Wt.T)
    out, loads, writes, ploads, pwrites = orc.tiled_matmul_count(A, Bm, g["block_M"], g["block_N"], g["block_K"])
    assert (loads, writes) == (g["total_load"], g["total_write"])
    assert (ploads, pwrites) == (g["total_load"], g["total_write"])  # tiles divide the shape
    assert np.allclose(out, A.astype(np.float64) @ Bm.astype(np.float64), rtol=1e-6, atol=0)
    Y, _ = orc.gemm_nt(A, Wt, "f32")
    assert np.max(np.abs(Y - out)) <= 2 * np.max(np.abs(Y)) * 2.0 ** -24


def pin_tiled_closed_forms(orc):
    cdiv = lambda a, b: -(-a // b)
    for (M, N, K, bm, bn, bk) in [(17, 10, 13, 5, 3, 6), (15, 9, 12, 5, 3, 6), (1, 1, 1, 4, 4, 4),
                                  (33, 21, 7, 8, 16, 4)]:
        g = np.random.default_rng(M + N + K)
        A = g.integers(-3, 4, (M, K)).astype(np.float32)
        Bm = g.integers(-3, 4, (K, N)).astype(np.float32)
        out, loads, writes, ploads, pwrites = orc.tiled_matmul_count(A, Bm, bm, bn, bk)
        assert loads == M * K * cdiv(N, bn) + K * N * cdiv(M, bm)
        assert writes == M * N
        assert ploads == (bm * bk + bk * bn) * cdiv(M, bm) * cdiv(N, bn) * cdiv(K, bk)
        assert pwrites == bm * bn * cdiv(M, bm) * cdiv(N, bn)
        assert np.array_equal(out, (A.astype(np.int64) @ Bm.astype(np.int64)).astype(np.float32))


# ----------------------------------------------------------- decode pins

def pin_decode_all_16bit(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype in ("bf16", "f16"):
        mine = orc.decode(pats, dtype)
        ref = lib_decode(pats, dtype)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan), dtype
        assert np.array_equal(mine[~nan], ref[~nan]), dtype


def pin_rejects_bad_arguments(orc):
    import ctypes
    lib = orc.lib
    buf = np.zeros(64, np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert lib.oracle_trimul_causal(p, p, None, 1, 2, 10, 3, 0) == -1   # C % NH != 0
    assert lib.oracle_trimul_causal(p, p, None, 1, 2, 12, 3, 7) == -1   # bad dtype
    assert lib.oracle_gemm_nt(p, p, p, None, 2, 2, 3, 2, 3, 2, 0) == -1  # ldx < K
    assert lib.oracle_trimul_causal(p, p, None, 0, 5, 12, 3, 0) == 0    # empty batch
    assert lib.oracle_causal_softmax(p, None, p, p, None, 1, 2, 12, 3, 0, 2) == -1  # bad mode
    assert lib.oracle_causal_softmax(p, None, p, p, None, 1, 2, 10, 3, 0, 1) == -1  # C % NH != 0


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
