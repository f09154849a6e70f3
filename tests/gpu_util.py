"""Shared helpers of the GPU parity tests: device copies of the seeded inputs,
guarded output buffers, and the element-by-element comparison against the
oracle at the tolerances of the contract:

  fp32 inputs:        |gpu - oracle| <= 1e-4 * sum|a_i b_i| + 1e-6
  bf16 / f16 inputs:  |gpu - oracle| <= 4e-3 * sum|a_i b_i|
  NaN mask:           bit-exact 0x7FC00000 above the diagonal
"""
from __future__ import annotations

import sys

import numpy as np

QNAN = 0x7FC00000
SENTINEL = -1                 # 0xFFFFFFFF: marks an element no kernel wrote
CANARY = 0x7F800001           # guard-band fill around every output
GUARD = 1024                  # elements of guard band on each side

TOL = {"f32": (1e-4, 1e-6), "bf16": (4e-3, 0.0), "f16": (4e-3, 0.0)}


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


def check_guards(buf, n: int) -> None:
    h = buf.cpu().numpy()
    assert np.all(h[:GUARD] == CANARY), "write before the output buffer"
    assert np.all(h[GUARD + n:] == CANARY), "write past the output buffer"


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
