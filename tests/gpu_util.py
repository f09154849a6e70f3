"""Shared helpers of the GPU parity tests: device copies of the seeded inputs,
guarded output buffers, and the element-by-element comparison against the
oracle at the tolerances of the contract:

  fp32 inputs:        |gpu - oracle| <= 1e-4 * sum|a_i b_i| + 1e-6
  bf16 / f16 inputs:  |gpu - oracle| <= 4e-3 * sum|a_i b_i|
  NaN mask:           bit-exact 0x7FC00000 above the diagonal

16-bit score outputs are the fp32 score rounded once more (nearest even), so
they get the fp32 allowance plus one rounding of that format: half an ulp,
2^-8 (bfloat16) or 2^-11 (binary16) of the magnitude, and for binary16 half
its smallest subnormal, 2^-25. Their mask is 0x7FC0 / 0x7E00, bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

QNAN = 0x7FC00000
SENTINEL = -1                 # 0xFFFFFFFF: marks an element no kernel wrote
CANARY = 0x7F800001           # guard-band fill around every output
GUARD = 1024                  # elements of guard band on each side

TOL = {"f32": (1e-4, 1e-6), "bf16": (4e-3, 0.0), "f16": (4e-3, 0.0)}
NAN16 = {"bf16": 0x7FC0, "f16": 0x7E00}
ROUND16 = {"bf16": (2.0 ** -8, 0.0), "f16": (2.0 ** -11, 2.0 ** -25)}
SENTINEL16 = -1               # 0xFFFF
CANARY16 = 0x7C01             # guard-band fill of 16-bit outputs


def case(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (not captured)."""
    print(f"[gpu-case] {msg}", file=sys.__stderr__, flush=True)


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).cuda()


def guarded_output(n: int):
    """A device buffer of n float32 outputs between two guard bands; the output
    elements start as the sentinel pattern."""
    import torch
    buf = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.int32, device="cuda")
    buf[GUARD:GUARD + n] = SENTINEL
    return buf, buf[GUARD:GUARD + n].view(torch.float32)


def guarded_output16(n: int, out_dtype: str):
    """n 16-bit outputs between guard bands, starting as the sentinel; returns
    (buffer, the n-element view as the output dtype)."""
    import torch
    buf = torch.full((n + 2 * GUARD,), CANARY16, dtype=torch.int16, device="cuda")
    buf[GUARD:GUARD + n] = SENTINEL16
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float16
    return buf, buf[GUARD:GUARD + n].view(tdt)


def check_guards(buf, n: int) -> None:
    import torch
    canary = CANARY16 if buf.dtype == torch.int16 else CANARY
    assert np.all(buf[:GUARD].cpu().numpy() == canary), "write before the output buffer"
    assert np.all(buf[GUARD + n:].cpu().numpy() == canary), "write past the output buffer"


def bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def assert_close(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, dtype: str, what: str) -> float:
    """Element-wise tolerance check; returns max(err / allowed)."""
    rel, ab = TOL[dtype]
    g = gpu.astype(np.float64)
    err = np.abs(g - ref.astype(np.float64))
    lim = rel * bound + ab
    bad = ~(err <= lim)  # NaN or an unwritten sentinel counts as bad
    if bad.any():
        idx = tuple(int(i) for i in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first {idx}: "
                             f"gpu={gpu[idx]!r} oracle={ref[idx]!r} bound={bound[idx]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(lim > 0, err / np.where(lim > 0, lim, 1), 0.0)
    return float(r.max()) if r.size else 0.0


def decode16(h: np.ndarray, out_dtype: str) -> np.ndarray:
    h = np.asarray(h).view(np.uint16)
    if out_dtype == "f16":
        return h.view(np.float16).astype(np.float64)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_scores16(gpu16: np.ndarray, ref: np.ndarray, bound: np.ndarray, in_dtype: str, out_dtype: str,
                    what: str, exact16: np.ndarray | None = None) -> float:
    """16-bit scores (raw uint16 patterns) against the oracle's fp32 scores:
    the mask bit-exact, the rest within the fp32 allowance plus one rounding to
    the 16-bit format -- or bit-exact to `exact16` (the oracle's rounding of
    exact fp32 scores) where given."""
    g = np.asarray(gpu16).view(np.uint16)
    mask = bits(ref) == QNAN
    if not np.all(g[mask] == NAN16[out_dtype]):
        raise AssertionError(f"{what}: {int(np.sum(g[mask] != NAN16[out_dtype]))} masked elements are not "
                             f"the {out_dtype} NaN pattern {NAN16[out_dtype]:#06x}")
    low = ~mask
    if exact16 is not None:
        if not np.array_equal(g[low], np.asarray(exact16)[low]):
            idx = tuple(int(i) for i in np.argwhere((g != exact16) & low)[0])
            raise AssertionError(f"{what}: not bit-exact; first {idx}: gpu={g[idx]:#06x} "
                                 f"oracle={int(exact16[idx]):#06x}")
        return 0.0
    dec = decode16(g[low], out_dtype)
    if not np.all(np.isfinite(dec)):
        raise AssertionError(f"{what}: non-finite value on or below the diagonal")
    rel, ab = TOL[in_dtype]
    r16, a16 = ROUND16[out_dtype]
    r = ref[low].astype(np.float64)
    fp32_allow = rel * bound[low] + ab
    lim = fp32_allow + r16 * (np.abs(r) + fp32_allow) + a16
    err = np.abs(dec - r)
    bad = ~(err <= lim)
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first: "
                             f"gpu={dec[i]!r} oracle={r[i]!r} allowed={lim[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(lim > 0, err / np.where(lim > 0, lim, 1), 0.0)
    return float(q.max()) if q.size else 0.0


def upper_mask(T: int) -> np.ndarray:
    """(T, T) booleans, True strictly above the diagonal (t2 > t)."""
    return np.triu(np.ones((T, T), dtype=bool), 1)


def _plane_check(ok: np.ndarray, err: np.ndarray, lim: np.ndarray, up: np.ndarray, got, ref, what: str) -> float:
    ok |= up
    if not ok.all():
        bad = ~ok
        t, t2 = (int(i) for i in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {int((~up).sum())} on or below the diagonal out of "
                             f"tolerance; first (t={t}, t2={t2}): gpu={got[t, t2]!r} oracle={ref[t, t2]!r} "
                             f"allowed={lim[t, t2]!r}")
    q = np.divide(err, lim, out=np.zeros_like(err), where=(lim > 0) & ~up)
    return float(q.max()) if q.size else 0.0


def assert_plane_scores(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, dtype: str, what: str,
                        up: np.ndarray) -> float:
    """One whole (T, T) plane of fp32 scores against the oracle's: the NaN
    pattern bit-exact exactly where t2 > t (`up`), every other element finite
    and within the tolerance (an unwritten sentinel is a NaN and fails).
    Returns max(err / allowed)."""
    gb = np.asarray(gpu, np.float32).view(np.uint32)
    is_mask = gb == QNAN
    if not np.array_equal(is_mask, up):
        raise AssertionError(f"{what}: {int(np.sum(is_mask != up))} elements where the NaN pattern 0x7FC00000 "
                             f"and the causal mask disagree")
    rel, ab = TOL[dtype]
    err = np.abs(gpu.astype(np.float64) - ref)
    lim = rel * bound + ab
    return _plane_check(err <= lim, err, lim, up, gpu, ref, what)


def assert_plane_scores16(gpu16: np.ndarray, ref: np.ndarray, bound: np.ndarray, in_dtype: str, out_dtype: str,
                          what: str, up: np.ndarray) -> float:
    """One whole (T, T) plane of 16-bit scores (raw uint16 patterns) against
    the oracle's fp32 scores: the 16-bit NaN pattern exactly where t2 > t, the
    rest finite and within the fp32 allowance plus one rounding of the format."""
    g = np.asarray(gpu16).view(np.uint16)
    is_mask = g == NAN16[out_dtype]
    if not np.array_equal(is_mask, up):
        raise AssertionError(f"{what}: {int(np.sum(is_mask != up))} elements where the {out_dtype} NaN pattern "
                             f"{NAN16[out_dtype]:#06x} and the causal mask disagree")
    rel, ab = TOL[in_dtype]
    r16, a16 = ROUND16[out_dtype]
    dec = decode16(g, out_dtype)
    fp32_allow = rel * bound + ab
    lim = fp32_allow + r16 * (np.abs(ref) + fp32_allow) + a16
    err = np.abs(dec - ref)
    return _plane_check(err <= lim, err, lim, up, dec, ref, what)


def assert_exact(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    if not np.array_equal(bits(gpu), bits(ref)):
        idx = tuple(int(i) for i in np.argwhere(bits(gpu) != bits(ref))[0])
        raise AssertionError(f"{what}: not bit-exact; first {idx}: gpu={gpu[idx]!r} oracle={ref[idx]!r}")


def assert_scores(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, dtype: str, what: str,
                  exact: bool = False) -> float:
    """Scores: NaN pattern bit-exact where the oracle has it, the rest finite
    and within tolerance (or bit-exact)."""
    mask = bits(ref) == QNAN
    gb = bits(gpu)
    if not np.array_equal(gb[mask], bits(ref)[mask]):
        n = int(np.sum(gb[mask] != QNAN))
        raise AssertionError(f"{what}: {n} masked elements are not the NaN pattern 0x7FC00000")
    low = ~mask
    if not np.all(np.isfinite(gpu[low])):
        raise AssertionError(f"{what}: non-finite value on or below the diagonal")
    if exact:
        assert_exact(gpu[low], ref[low], what)
        return 0.0
    return assert_close(gpu[low], ref[low], bound[low], dtype, what)


# ------------------------------------------------------------------ softmax
#
# Tolerance of the causal softmax, derived from the score tolerance above.
# Let d_j be the allowance of score j of a row (the contract's, plus half an
# fp32 ulp of the score since the oracle's softmax uses unrounded scores;
# 0 where the scores are exact) and D = max_{j <= t} d_j. The row maximum and
# log-sum-exp are 1-Lipschitz in the largest score error, so
#   |row_max - m|           <= D
#   |(x_j - m^) - L^ - lp_j| <= d_j + D + S + R (1 + |lp_j| + |L|)
#   |row_logsum - L|        <= 2 D + S + R (1 + |L|)
# with S = (n + 64) 2^-24 the fp32 summation of n = t + 1 terms (exp2 and
# rescaling included) and R = 2^-21 the roundings of log2, ln 2 and the two
# subtractions. A probability p = exp(lp) is then within p expm1(that + R(1 +
# |lp|)), and at least 2^-126 (results below fp32's normal range may flush
# to zero). The kernels form p as exp2(fma(fma(a, scale, -max), log2 e,
# -logsum log2 e)): its roundings, and exp2's own, come to at most
# 2^-24 (2 + 5 |lp|) in ln p (logsum <= |lp| since x <= max and logsum >= 0),
# inside the R (1 + 2 |lp|) left for that step. 16-bit outputs add one
# rounding of the format, as for the scores.

FILL = {("f32", "log"): 0xFF800000, ("f32", "prob"): 0x00000000,
        ("bf16", "log"): 0xFF80, ("f16", "log"): 0xFC00, ("bf16", "prob"): 0x0000, ("f16", "prob"): 0x0000}
SM_R = 2.0 ** -21


def softmax_allowance(bound: np.ndarray, t_idx: np.ndarray, in_dtype: str, exact_scores: bool = False):
    """(d (R, T), D (R,), S (R,), valid (R, T)) for rows of index t_idx."""
    rel, ab = TOL[in_dtype]
    T = bound.shape[-1]
    valid = np.arange(T)[None, :] <= np.asarray(t_idx)[:, None]
    if exact_scores:
        d = np.zeros(bound.shape)
    else:
        d = np.where(valid, rel * bound + ab + 2.0 ** -24 * bound, 0.0)
    return d, d.max(axis=1), (np.asarray(t_idx) + 65) * 2.0 ** -24, valid


def _ratio(err, lim):
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(lim > 0, err / np.where(lim > 0, lim, 1), np.where(err > 0, np.inf, 0.0))
    return float(q.max()) if q.size else 0.0


def assert_softmax_stats(mx, ls, mx_ref, ls_ref, bound, t_idx, in_dtype, what, exact_scores=False,
                         extra=0.0) -> float:
    """GPU row statistics (R,) against the oracle's. extra: a further
    allowance on row_logsum (per row or scalar)."""
    _, D, S, _ = softmax_allowance(bound, t_idx, in_dtype, exact_scores)
    mx, ls = np.asarray(mx, np.float64), np.asarray(ls, np.float64)
    em, lm = np.abs(mx - mx_ref), D
    el, ll = np.abs(ls - ls_ref), 2 * D + S + SM_R * (1 + np.abs(ls_ref)) + extra
    for name, e, lim, g, r in (("row_max", em, lm, mx, mx_ref), ("row_logsum", el, ll, ls, ls_ref)):
        bad = ~(e <= lim)
        if bad.any():
            i = int(np.argwhere(bad)[0][0])
            raise AssertionError(f"{what}: {name} {int(bad.sum())} of {bad.size} out of tolerance; first row "
                                 f"{i} (t={int(t_idx[i])}): gpu={g[i]!r} oracle={r[i]!r} allowed={lim[i]!r}")
    return max(_ratio(em, lm), _ratio(el, ll))


def prob_limits(ref, ls_ref, bound, t_idx, in_dtype, exact_scores=False):
    """Allowed |p_gpu - p| per element (rows (R, T) of fp32 probabilities),
    and the mask of entries t2 <= t."""
    d, D, S, valid = softmax_allowance(bound, t_idx, in_dtype, exact_scores)
    lsr = np.broadcast_to(np.abs(np.asarray(ls_ref))[:, None], ref.shape)
    lp = np.log(np.maximum(ref, 1e-300))
    tl = d + D[:, None] + S[:, None] + SM_R * (1 + np.abs(lp) + lsr)
    rel = np.where(valid, np.expm1(tl + SM_R * (1 + np.abs(lp))), 0.0)
    require_pinning(rel, t_idx, "probabilities")
    return np.where(valid, ref * rel + 2.0 ** -126, 0.0), valid


def require_pinning(rel, t_idx, what: str) -> None:
    """The probability bounds are relative: p_gpu within p (1 +- rel). Where a
    row's score allowances make rel reach 1/2 (saturated random rows: a
    relative allowance on scores in the thousands moves exp by orders of
    magnitude) the bound pins no value. Such rows fail here instead of passing
    on a void bound; their values are tested with exact scores (ramp rows)."""
    rel = np.asarray(rel)
    if rel.size and not np.all(rel < 0.5):
        i = int(np.argmax(rel.max(axis=-1)))
        raise AssertionError(f"{what}: the score allowances of row {i} (t={int(np.asarray(t_idx)[i])}) allow a "
                             f"relative error of {float(rel[i].max()):.3g}: the bound pins no value "
                             f"(use exact scores)")


def assert_attention(got, ref, absw, p_ref, ls_ref, bound, t_idx, v_abs, in_dtype, what, exact_scores=False) -> float:
    """Attention output rows (R, HS) of one head against the oracle's. Each
    output is sum_j p_j v_j: with |p_gpu - p| <= lim_j (prob_limits) and an
    fp32 sum of n products, |y_gpu - y| <= sum_j lim_j |v_j| + S sum_j p_j |v_j|
    (S as for the softmax); v_abs is |V| (T, HS) of the head. For 16-bit
    inputs p is rounded to the input format before the products: one more
    relative rounding of that format on p_gpu, and 2^-126 for a flushed one."""
    lim_p, valid = prob_limits(p_ref, ls_ref, bound, t_idx, in_dtype, exact_scores)
    if in_dtype != "f32":
        r16, a16 = ROUND16[in_dtype]
        lim_p = lim_p + np.where(valid, r16 * (p_ref + lim_p) + max(a16, 2.0 ** -126), 0.0)
    S = (np.asarray(t_idx) + 65) * 2.0 ** -24
    lim = lim_p @ v_abs + S[:, None] * absw
    g = np.asarray(got, np.float64)
    if not np.all(np.isfinite(g)):
        raise AssertionError(f"{what}: non-finite output")
    err = np.abs(g - ref)
    bad = ~(err <= lim)
    if bad.any():
        i, j = (int(x) for x in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first (row {i}, col {j}): "
                             f"gpu={g[i, j]!r} oracle={ref[i, j]!r} allowed={lim[i, j]!r}")
    return _ratio(err, lim)


# Single-pass attention (cas_causal_attention_fused). The kernel forms
# y = sum_j w_j v_j / sum_j w_j with w_j = exp2(a_j c - ms) against a running
# offset ms that lags the running maximum by at most ONLINE_TAU in base 2 and
# rescales earlier terms by exp2(ms_old - ms_new) when it moves (at most once
# per 64-key step). An error common to all w_j cancels in the ratio. Per
# weight, in ln w_j, there remain the score error d_j, the roundings of the
# exp2 argument and of exp2 itself, 2^-24 (8 + 3 (|lp_j| + |L| + TAU ln 2)),
# and 2^-22 per rescale. With E_j = expm1(that) and E = max_j E_j the
# normalised weights are within pi_j (E_j + E) / (1 - E), so
#   |y_gpu - y| <= sum_j lim_j |v_j| + (u16 + 2 S + 2^-22) (sum_j p_j |v_j| + sum_j lim_j |v_j|) + a16 sum_j |v_j|,
# where u16 and a16 are the input format's rounding of w_j for the 16-bit
# MFMA (the sum uses the unrounded w_j), S the fp32 sums, and 2^-22 the final
# division; weights that flush to zero are below 2^-126 of the sum. The bound
# needs E < 1/2; a row with larger score allowances (saturated random 16-bit
# rows, where a 4e-3 relative allowance on scores in the hundreds moves the
# weights by orders of magnitude) pins no value, so such rows fail here
# rather than pass on a looser bound: saturated rows are tested with exact
# scores (ramp rows) instead. The row_logsum adds 2^-22 per step and 2^-21 TAU
# (the offset's distance from the maximum) to the two-pass allowance; row_max
# is the two-pass value.
ONLINE_TAU = 8.0


def online_steps(t_idx):
    return np.asarray(t_idx) // 64 + 1


def assert_attention_online(got, ref, absw, p_ref, ls_ref, bound, t_idx, v_abs, in_dtype, what,
                            exact_scores=False) -> float:
    d, _, S, valid = softmax_allowance(bound, t_idx, in_dtype, exact_scores)
    lp = np.log(np.maximum(p_ref, 1e-300))
    L = np.abs(np.asarray(ls_ref, np.float64))[:, None]
    arg = d + 2.0 ** -24 * (8 + 3 * (np.abs(lp) + L + ONLINE_TAU * np.log(2.0))) + \
        online_steps(t_idx)[:, None] * 2.0 ** -22
    E = np.where(valid, np.expm1(arg), 0.0)
    Em = E.max(axis=1, keepdims=True)
    lim_p = np.where(valid, p_ref * (E + Em) / (1 - Em) + 2.0 ** -118, 0.0)
    u16, a16 = ROUND16[in_dtype] if in_dtype != "f32" else (0.0, 0.0)
    lpv = lim_p @ v_abs
    vsum = valid.astype(np.float64) @ v_abs
    lim = lpv + (u16 + 2 * S[:, None] + 2.0 ** -22) * (absw + lpv) + a16 * vsum
    if not np.all(Em < 0.5):
        i = int(np.argmax(Em[:, 0]))
        raise AssertionError(f"{what}: the score allowances of row {i} (t={int(np.asarray(t_idx)[i])}) move its "
                             f"weights by up to {float(Em[i, 0]):.3g}: the bound pins no value (use exact scores)")
    g = np.asarray(got, np.float64)
    if not np.all(np.isfinite(g)):
        raise AssertionError(f"{what}: non-finite output")
    err = np.abs(g - ref)
    bad = ~(err <= lim)
    if bad.any():
        i, j = (int(x) for x in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first (row {i}, col {j}): "
                             f"gpu={g[i, j]!r} oracle={ref[i, j]!r} allowed={lim[i, j]!r}")
    return _ratio(err, lim)


def online_logsum_extra(t_idx):
    return online_steps(t_idx) * 2.0 ** -22 + SM_R * ONLINE_TAU


def assert_softmax(got, ref, ls_ref, bound, t_idx, in_dtype, mode, out_dtype, what, exact_scores=False) -> float:
    """GPU softmax rows (R, T) against the oracle's (float64): float32 values
    for fp32 output, raw uint16 patterns for 16-bit output. The masked part
    (t2 > t) must be the fill pattern bit for bit."""
    d, D, S, valid = softmax_allowance(bound, t_idx, in_dtype, exact_scores)
    if out_dtype == "f32":
        gb = np.asarray(got, np.float32).view(np.uint32)
        vals = np.asarray(got, np.float32).astype(np.float64)
    else:
        gb = np.asarray(got).view(np.uint16)
        vals = decode16(gb, out_dtype)
    fill = FILL[(out_dtype, mode)]
    if not np.all(gb[~valid] == fill):
        n = int(np.sum(gb[~valid] != fill))
        raise AssertionError(f"{what}: {n} masked elements are not the fill pattern {fill:#x}")
    lsr = np.broadcast_to(np.abs(np.asarray(ls_ref))[:, None], ref.shape)
    if mode == "log":
        lim = d + D[:, None] + S[:, None] + SM_R * (1 + np.abs(ref) + lsr)
    else:
        lp = np.log(np.maximum(ref, 1e-300))
        tl = d + D[:, None] + S[:, None] + SM_R * (1 + np.abs(lp) + lsr)
        rel = np.where(valid, np.expm1(tl + SM_R * (1 + np.abs(lp))), 0.0)
        require_pinning(rel, t_idx, what)
        lim = ref * rel + 2.0 ** -126
    if out_dtype != "f32":
        r16, a16 = ROUND16[out_dtype]
        lim = lim + r16 * (np.abs(ref) + lim) + a16
    v, r, lm = vals[valid], ref[valid], lim[valid]
    if not np.all(np.isfinite(v)):
        raise AssertionError(f"{what}: non-finite value on or below the diagonal")
    err = np.abs(v - r)
    bad = ~(err <= lm)
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        rows, cols = np.nonzero(valid)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first (row {rows[i]}, "
                             f"t2 {cols[i]}): gpu={v[i]!r} oracle={r[i]!r} allowed={lm[i]!r}")
    return _ratio(err, lm)
