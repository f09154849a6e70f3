"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
element by element on the same seeded inputs.

Sizes span several tiles and ragged tails; the workload tests run the
full-size configurations in the launch configuration the benchmark times and
compare every element of every output with the oracle's, each output starting
as a sentinel between guard bands."""
import numpy as np
import pytest
import torch

import causal_attention_score_amd as cas
from causal_attention_score_amd import synth
from gpu_util import (SENTINEL, assert_close, assert_exact, assert_plane_scores, assert_plane_scores16,
                      assert_scores, assert_scores16, case, check_guards, guarded_output, guarded_output16,
                      to_device, upper_mask)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "f16"]


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def run_gemm(X, W, dtype, M, N, K, label, ldy=None):
    ldy = N if ldy is None else ldy
    n = M * ldy
    buf, flat = guarded_output(n)
    y = flat.view(M, ldy)[:, :N]
    case(f"{label} gemm_nt {dtype} M={M} N={N} K={K} ldy={ldy}")
    cas.gemm_nt(to_device(X, dtype), to_device(W, dtype), out=y)
    torch.cuda.synchronize()
    check_guards(buf, n)
    return flat.view(M, ldy).cpu().numpy()


# ------------------------------------------------------------------ gemm_nt

GEMM_SHAPES = [(1, 1, 1), (2, 3, 7), (7, 15, 31), (15, 9, 12), (33, 63, 65), (65, 33, 127), (127, 129, 255),
               (129, 127, 257), (255, 257, 33), (257, 255, 770), (1, 257, 129), (300, 1, 64), (64, 64, 64),
               (128, 128, 128), (96, 160, 770), (200, 72, 3)]


@pytest.mark.parametrize("tile", ["64", "128"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_ragged(orc, monkeypatch, shape, dtype, tile):
    monkeypatch.setenv("CAS_GEMM_TILE", tile)
    M, N, K = shape
    X, W = synth.gemm_inputs(M, N, K, dtype, seed=M * 7 + N * 3 + K)
    ref, bound = orc.gemm_nt(X, W, dtype)
    y = run_gemm(X, W, dtype, M, N, K, f"tile{tile}")
    assert_close(y, ref, bound, dtype, f"gemm {shape} {dtype} tile{tile}")


# 256 x 256 tiles with loads straight into LDS (16-bit inputs, K a multiple of
# 8): ragged M and N, K not a multiple of the 64-element chunk, one chunk, and
# shapes with several tiles per dimension.
WIDE_SHAPES = [(256, 256, 64), (300, 520, 136), (257, 255, 8), (513, 260, 264), (1, 300, 72), (600, 40, 1000),
               (520, 513, 4104), (255, 1, 16), (768, 512, 192)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_wide_ragged(orc, monkeypatch, shape, dtype):
    monkeypatch.setenv("CAS_GEMM_TILE", "256")
    M, N, K = shape
    X, W = synth.gemm_inputs(M, N, K, dtype, seed=M * 5 + N * 11 + K)
    ref, bound = orc.gemm_nt(X, W, dtype)
    y = run_gemm(X, W, dtype, M, N, K, "tile256")
    assert_close(y, ref, bound, dtype, f"gemm wide {shape} {dtype}")


# 16-bit rows not in 16-byte pieces on 256 x 256 tiles: K not a multiple of 8
# (the wide kernel over the first K - K % 8 columns, a tail kernel adding the
# rest), row pitches above K, and bases one element off a 16-byte boundary.
# (M, N, K, base offset in elements, pitch padding in elements)
WIDE_UNALIGNED = [(300, 520, 771, 0, 0), (257, 255, 9, 0, 0), (600, 40, 1023, 1, 3), (513, 260, 264, 1, 1),
                  (256, 256, 130, 0, 5), (1024, 1024, 1023, 0, 0), (520, 513, 4097, 0, 0), (64, 300, 15, 1, 0)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", WIDE_UNALIGNED, ids=lambda s: "x".join(map(str, s)))
def test_gemm_wide_unaligned(orc, monkeypatch, shape, dtype):
    monkeypatch.setenv("CAS_GEMM_TILE", "256")
    M, N, K, off, pad = shape
    ldx, ldw = K + pad, K + pad + 2
    g = np.random.default_rng(M * 7 + N * 3 + K)
    Xf = synth.to_storage(g.standard_normal((M * ldx + off,)).astype(np.float32), dtype)
    Wf = synth.to_storage(g.standard_normal((N * ldw + off,)).astype(np.float32), dtype)
    ref, bound = orc.gemm_nt(Xf[off:], Wf[off:], dtype, M=M, N=N, K=K, ldx=ldx, ldw=ldw, ldy=N)
    dx, dw = to_device(Xf, dtype), to_device(Wf, dtype)
    x = dx[off:].as_strided((M, K), (ldx, 1))
    w = dw[off:].as_strided((N, K), (ldw, 1))
    buf, flat = guarded_output(M * N)
    case(f"gemm wide unaligned {shape} {dtype}")
    cas.gemm_nt(x, w, out=flat.view(M, N))
    torch.cuda.synchronize()
    check_guards(buf, M * N)
    assert_close(flat.view(M, N).cpu().numpy(), ref, bound, dtype, f"gemm wide unaligned {shape} {dtype}")


# The 128 x 128 register ring for K not a multiple of its 16-byte pieces: the
# ring over the first K - K % (16 / es) columns, then the tail kernel; pitches
# above K and bases one element off a 16-byte boundary.
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(300, 520, 771, 0, 0), (257, 255, 9, 1, 3), (129, 300, 130, 1, 0),
                                   (640, 384, 1023, 0, 1)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_ring128_ktail(orc, monkeypatch, shape, dtype):
    monkeypatch.setenv("CAS_GEMM_TILE", "128")
    M, N, K, off, pad = shape
    ldx, ldw = K + pad, K + pad + 1
    g = np.random.default_rng(M * 5 + N * 7 + K)
    Xf = synth.to_storage(g.standard_normal((M * ldx + off,)).astype(np.float32), dtype)
    Wf = synth.to_storage(g.standard_normal((N * ldw + off,)).astype(np.float32), dtype)
    ref, bound = orc.gemm_nt(Xf[off:], Wf[off:], dtype, M=M, N=N, K=K, ldx=ldx, ldw=ldw, ldy=N)
    dx, dw = to_device(Xf, dtype), to_device(Wf, dtype)
    x = dx[off:].as_strided((M, K), (ldx, 1))
    w = dw[off:].as_strided((N, K), (ldw, 1))
    buf, flat = guarded_output(M * N)
    case(f"gemm ring128 k-tail {shape} {dtype}")
    cas.gemm_nt(x, w, out=flat.view(M, N))
    torch.cuda.synchronize()
    check_guards(buf, M * N)
    assert_close(flat.view(M, N).cpu().numpy(), ref, bound, dtype, f"gemm ring128 k-tail {shape} {dtype}")


# K a multiple of 128 (whole turns of the four-stage ring): the full-turn
# kernel, whose fetch has no per-chunk predicate; ragged M and N, one turn
# (K = 128) and several.
WIDE_FULL_SHAPES = [(300, 520, 256), (513, 260, 128), (256, 256, 512), (520, 513, 1024), (1, 300, 256),
                    (600, 40, 384), (257, 255, 640), (768, 512, 4096)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", WIDE_FULL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_wide_full_turns(orc, monkeypatch, shape, dtype):
    monkeypatch.setenv("CAS_GEMM_TILE", "256")
    M, N, K = shape
    X, W = synth.gemm_inputs(M, N, K, dtype, seed=M * 3 + N * 13 + K)
    ref, bound = orc.gemm_nt(X, W, dtype)
    y = run_gemm(X, W, dtype, M, N, K, "tile256 full turns")
    assert_close(y, ref, bound, dtype, f"gemm wide full turns {shape} {dtype}")


@pytest.mark.parametrize("shape", [(300, 520, 256), (520, 513, 1024)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_wide_full_turns_match_the_ring_kernel(monkeypatch, shape):
    """The full-turn kernel issues the ring kernel's MFMAs in the same order
    on the same fragments: the outputs are equal bit for bit."""
    monkeypatch.setenv("CAS_GEMM_TILE", "256")
    M, N, K = shape
    X, W = synth.gemm_inputs(M, N, K, "bf16", seed=5)
    full = run_gemm(X, W, "bf16", M, N, K, "full turns")
    monkeypatch.setenv("CAS_GEMM_WIDE", "ring")
    ring = run_gemm(X, W, "bf16", M, N, K, "ring")
    assert_exact(full, ring, f"full turns vs ring {shape}")


@pytest.mark.parametrize("layout", ["64x4", "128x2", "64x3", "128x2w8", "64x3w8", "ring"])
@pytest.mark.parametrize("shape", [(300, 520, 136), (520, 513, 1032)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_wide_tuning_layouts(orc, monkeypatch, shape, layout):
    """The wide kernel's other chunk widths, stage counts and wave layouts
    (CAS_GEMM_WIDE, tuning): four waves of 128 x 128 and eight of 128 x 64."""
    monkeypatch.setenv("CAS_GEMM_TILE", "256")
    monkeypatch.setenv("CAS_GEMM_WIDE", layout)
    M, N, K = shape
    X, W = synth.gemm_inputs(M, N, K, "bf16", seed=M + N + K)
    ref, bound = orc.gemm_nt(X, W, "bf16")
    y = run_gemm(X, W, "bf16", M, N, K, f"wide {layout}")
    assert_close(y, ref, bound, "bf16", f"gemm wide {layout} {shape}")


def test_gemm_wide_k0_writes_zeros(monkeypatch):
    monkeypatch.setenv("CAS_GEMM_TILE", "256")
    x = torch.empty((300, 0), device="cuda", dtype=torch.bfloat16)
    w = torch.empty((260, 0), device="cuda", dtype=torch.bfloat16)
    buf, flat = guarded_output(300 * 260)
    case("gemm wide K=0")
    cas.gemm_nt(x, w, out=flat.view(300, 260))
    torch.cuda.synchronize()
    check_guards(buf, 300 * 260)
    assert np.all(flat.cpu().numpy() == 0)


# The local-padding A/B baseline: the same product with the bounds checks
# kept inside the MFMA loop (CAS_VARIANT=predicated) must give the same results.
PRED_SHAPES = [(15, 9, 12), (65, 33, 127), (129, 127, 257), (257, 255, 770), (200, 72, 3), (1, 257, 129),
               (96, 160, 770)]


@pytest.mark.parametrize("tile", ["64", "128"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", PRED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_predicated_ragged(orc, monkeypatch, shape, dtype, tile):
    monkeypatch.setenv("CAS_VARIANT", "predicated")
    monkeypatch.setenv("CAS_GEMM_TILE", tile)
    M, N, K = shape
    X, W = synth.gemm_inputs(M, N, K, dtype, seed=M * 7 + N * 3 + K)
    ref, bound = orc.gemm_nt(X, W, dtype)
    y = run_gemm(X, W, dtype, M, N, K, f"predicated tile{tile}")
    assert_close(y, ref, bound, dtype, f"gemm predicated {shape} {dtype} tile{tile}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_predicated_exact_small_integers(orc, monkeypatch, dtype):
    monkeypatch.setenv("CAS_VARIANT", "predicated")
    for (M, N, K) in [(131, 67, 770), (300, 257, 1024)]:
        X, W = synth.gemm_inputs(M, N, K, dtype, seed=K + 1, dist="int")
        ref, _ = orc.gemm_nt(X, W, dtype)
        y = run_gemm(X, W, dtype, M, N, K, "predicated exact")
        assert_exact(y, ref, f"gemm predicated exact {(M, N, K)} {dtype}")


@pytest.mark.parametrize("tile", ["64", "128", "256"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_exact_small_integers(orc, monkeypatch, dtype, tile):
    """Integer inputs: every partial sum is an exact integer, so the GPU must
    equal the oracle bit for bit whatever its summation order."""
    monkeypatch.setenv("CAS_GEMM_TILE", tile)
    for (M, N, K) in [(131, 67, 770), (64, 256, 129), (5, 300, 1000), (300, 257, 1024)]:
        X, W = synth.gemm_inputs(M, N, K, dtype, seed=K, dist="int")
        ref, _ = orc.gemm_nt(X, W, dtype)
        y = run_gemm(X, W, dtype, M, N, K, "exact")
        assert_exact(y, ref, f"gemm exact {(M, N, K)} {dtype}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_strided_misaligned(orc, dtype):
    """Row pitches above K, bases one element off 16-byte alignment, and an
    output pitch above N: the narrow-load variants and the writeback mask."""
    M, N, K = 77, 45, 130
    ldx, ldw, ldy = K + 3, K + 5, N + 7
    g = np.random.default_rng(99)
    Xf = synth.to_storage(g.standard_normal((M * ldx + 1,)).astype(np.float32), dtype)
    Wf = synth.to_storage(g.standard_normal((N * ldw + 1,)).astype(np.float32), dtype)
    ref, bound = orc.gemm_nt(Xf[1:], Wf[1:], dtype, M=M, N=N, K=K, ldx=ldx, ldw=ldw, ldy=ldy)
    dx, dw = to_device(Xf, dtype), to_device(Wf, dtype)
    x = dx[1:].as_strided((M, K), (ldx, 1))
    w = dw[1:].as_strided((N, K), (ldw, 1))
    buf, flat = guarded_output(M * ldy)
    y = flat.view(M, ldy)[:, :N]
    case(f"gemm strided/misaligned {dtype}")
    cas.gemm_nt(x, w, out=y)
    torch.cuda.synchronize()
    check_guards(buf, M * ldy)
    h = flat.view(M, ldy).cpu().numpy()
    assert np.all(h[:, N:].view(np.int32) == SENTINEL), "wrote past N inside the output pitch"
    assert_close(h[:, :N], ref[:, :N], bound[:, :N], dtype, "gemm strided")


# fp32 on 64 x 64 tiles with loads straight into LDS: K below, at and just
# past one 32-float chunk, K % 4 != 0 (a 16-byte piece straddles K and reads
# past the row), row pitches even (8-byte-aligned rows) and odd (4-byte
# aligned: the load unit takes the pieces at any element alignment), and
# padding that holds NaN, which must not reach the products. The
# register-ring engine (CAS_GEMM_F32=ring) forms the same products in the
# same order: bit for bit.
DIRECT_SHAPES = [(1, 1, 2), (70, 90, 98), (64, 64, 32), (65, 63, 34), (130, 200, 96), (257, 255, 770),
                 (40, 300, 1026), (1, 1, 1), (65, 63, 33), (257, 255, 771), (40, 300, 1025)]


@pytest.mark.parametrize("pitch", ["even", "odd"])
@pytest.mark.parametrize("shape", DIRECT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_direct_nan_padding_and_ring(orc, monkeypatch, shape, pitch):
    M, N, K = shape
    if pitch == "even":
        ldx, ldw = (K + 2, K + 6) if K % 2 == 0 else (K + 1, K + 5)
    else:
        ldx, ldw = (K + 1, K + 3) if K % 2 == 0 else (K, K + 2)
    g = np.random.default_rng(M * 31 + K)
    Xf = np.full(M * ldx, np.nan, np.float32)
    Wf = np.full(N * ldw, np.nan, np.float32)
    Xf.reshape(M, ldx)[:, :K] = g.standard_normal((M, K))
    Wf.reshape(N, ldw)[:, :K] = g.standard_normal((N, K))
    ref, bound = orc.gemm_nt(Xf, Wf, "f32", M=M, N=N, K=K, ldx=ldx, ldw=ldw, ldy=N)
    x = to_device(Xf, "f32").as_strided((M, K), (ldx, 1))
    w = to_device(Wf, "f32").as_strided((N, K), (ldw, 1))
    got = {}
    for engine in ("direct", "ring"):
        if engine == "ring":
            monkeypatch.setenv("CAS_GEMM_F32", "ring")
        buf, flat = guarded_output(M * N)
        case(f"gemm fp32 {engine} {shape} NaN pitch padding")
        cas.gemm_nt(x, w, out=flat.view(M, N))
        torch.cuda.synchronize()
        check_guards(buf, M * N)
        got[engine] = flat.view(M, N).cpu().numpy()
    assert_close(got["direct"], ref, bound, "f32", f"gemm direct {shape}")
    assert np.array_equal(got["direct"].view(np.uint32), got["ring"].view(np.uint32)), "direct and ring differ"


@pytest.mark.parametrize("tile,ldx", [("64", 8_000_000), ("64", 9_000_000), ("128", 4_000_000), ("128", 4_500_000)])
def test_gemm_huge_row_pitch(orc, monkeypatch, tile, ldx):
    """Row pitches near the 31-bit offset range: the register-ring loop
    fetches through buffer offsets from a tile's first row while a tile's rows
    of the pitch fit below 2^31 bytes (64x64 tiles: 8M fp32 elements; 128x128
    tiles: 4M), and the two-stage loop takes over above that (9M; 4.5M). K and
    the pitch are multiples of four, so the loads are 16 bytes wide, the case
    in which 128x128 tiles take the ring too. Both must match the oracle."""
    monkeypatch.setenv("CAS_GEMM_TILE", tile)
    M, N, K = 3, 70, 100
    g = np.random.default_rng(ldx % 997)
    Xf = synth.to_storage(g.standard_normal(((M - 1) * ldx + K,)).astype(np.float32), "f32")
    W = synth.to_storage(g.standard_normal((N, K)).astype(np.float32), "f32")
    ref, bound = orc.gemm_nt(Xf, W.ravel(), "f32", M=M, N=N, K=K, ldx=ldx, ldw=K, ldy=N)
    x = to_device(Xf, "f32").as_strided((M, K), (ldx, 1))
    buf, flat = guarded_output(M * N)
    case(f"gemm tile {tile} row pitch {ldx}")
    cas.gemm_nt(x, to_device(W, "f32"), out=flat.view(M, N))
    torch.cuda.synchronize()
    check_guards(buf, M * N)
    assert_close(flat.view(M, N).cpu().numpy(), ref, bound, "f32", f"gemm tile {tile} ldx={ldx}")


# ------------------------------------------------------- batch_matmul_nt

BMM_SHAPES = [(192, 120, 120, 64), (3, 65, 33, 127), (5, 1, 257, 129), (7, 200, 72, 3), (2, 128, 128, 128),
              (4, 15, 9, 12)]


def run_bmm(X, W, dtype, label):
    Bt, M, K = X.shape
    N = W.shape[1]
    n = Bt * M * N
    buf, flat = guarded_output(n)
    case(f"{label} batch_matmul_nt {dtype} batch={Bt} M={M} N={N} K={K}")
    cas.batch_matmul_nt(to_device(X, dtype), to_device(W, dtype), out=flat.view(Bt, M, N))
    torch.cuda.synchronize()
    check_guards(buf, n)
    return flat.view(Bt, M, N).cpu().numpy()


@pytest.mark.parametrize("tile", ["64", "128"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", BMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bmm_ragged(orc, monkeypatch, shape, dtype, tile):
    monkeypatch.setenv("CAS_GEMM_TILE", tile)
    Bt, M, N, K = shape
    X, W = synth.gemm_inputs(Bt * M, Bt * N, K, dtype, seed=Bt + M + N + K)
    X, W = X.reshape(Bt, M, K), W.reshape(Bt, N, K)
    ref, bound = orc.batch_matmul_nt(X, W, dtype)
    y = run_bmm(X, W, dtype, f"tile{tile}")
    assert_close(y, ref, bound, dtype, f"bmm {shape} {dtype} tile{tile}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_bmm_predicated(orc, monkeypatch, dtype):
    monkeypatch.setenv("CAS_VARIANT", "predicated")
    Bt, M, N, K = 24, 120, 120, 64
    X, W = synth.gemm_inputs(Bt * M, Bt * N, K, dtype, seed=31)
    X, W = X.reshape(Bt, M, K), W.reshape(Bt, N, K)
    ref, bound = orc.batch_matmul_nt(X, W, dtype)
    y = run_bmm(X, W, dtype, "predicated")
    assert_close(y, ref, bound, dtype, f"bmm predicated {dtype}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_bmm_strides_and_broadcast(orc, dtype):
    """Batch strides above one block, odd row pitches, one W block for every
    batch (stride 0), and an output batch stride that leaves gaps: the gaps
    and the pitch padding keep their sentinel."""
    Bt, M, N, K = 5, 37, 29, 50
    ldx, ldw, ldy = K + 3, K + 1, N + 5
    bsx, bsy = M * ldx + 7, M * ldy + 11
    g = np.random.default_rng(7)
    Xf = synth.to_storage(g.standard_normal((Bt * bsx,)).astype(np.float32), dtype)
    Wf = synth.to_storage(g.standard_normal((N * ldw,)).astype(np.float32), dtype)
    Xb = np.stack([Xf[b * bsx:b * bsx + M * ldx].reshape(M, ldx)[:, :K] for b in range(Bt)])
    Wb = np.stack([Wf.reshape(N, ldw)[:, :K]] * Bt)
    ref, bound = orc.batch_matmul_nt(np.ascontiguousarray(Xb), np.ascontiguousarray(Wb), dtype)
    dx, dw = to_device(Xf, dtype), to_device(Wf, dtype)
    x = dx.as_strided((Bt, M, K), (bsx, ldx, 1))
    w = dw.as_strided((Bt, N, K), (0, ldw, 1))
    n = Bt * bsy
    buf, flat = guarded_output(n)
    y = flat.as_strided((Bt, M, N), (bsy, ldy, 1))
    case(f"bmm strides/broadcast {dtype}")
    cas.batch_matmul_nt(x, w, out=y)
    torch.cuda.synchronize()
    check_guards(buf, n)
    h = flat.cpu().numpy()
    got = np.stack([h[b * bsy:b * bsy + M * ldy].reshape(M, ldy)[:, :N] for b in range(Bt)])
    assert_close(got, ref, bound, dtype, "bmm strides")
    mask = np.ones(n, dtype=bool)
    for b in range(Bt):
        for m in range(M):
            mask[b * bsy + m * ldy:b * bsy + m * ldy + N] = False
    assert np.all(h[mask].view(np.int32) == SENTINEL), "wrote outside the output blocks"


def test_bmm_k0_and_empty():
    x = torch.empty((3, 5, 0), device="cuda")
    w = torch.empty((3, 7, 0), device="cuda")
    buf, flat = guarded_output(105)
    case("bmm K=0")
    cas.batch_matmul_nt(x, w, out=flat.view(3, 5, 7))
    torch.cuda.synchronize()
    check_guards(buf, 105)
    assert np.all(flat.cpu().numpy() == 0)
    assert cas.batch_matmul_nt(torch.zeros((0, 4, 8), device="cuda"), torch.zeros((0, 3, 8), device="cuda")).shape == (0, 4, 3)


def test_gemm_k0_writes_zeros():
    x = torch.empty((5, 0), device="cuda")
    w = torch.empty((7, 0), device="cuda")
    buf, flat = guarded_output(35)
    case("gemm K=0")
    cas.gemm_nt(x, w, out=flat.view(5, 7))
    torch.cuda.synchronize()
    check_guards(buf, 35)
    assert np.all(flat.cpu().numpy() == 0)


def test_gemm_empty_is_noop():
    x = torch.zeros((0, 4), device="cuda")
    w = torch.zeros((3, 4), device="cuda")
    y = cas.gemm_nt(x, w)
    assert y.shape == (0, 3)


def test_gemm_alias_rejected():
    buf = torch.zeros(4096, device="cuda")
    x = buf[:64].view(8, 8)
    w = buf[64:128].view(8, 8)
    with pytest.raises(cas.CasError) as e:
        cas.gemm_nt(x, w, out=buf[32:96].view(8, 8))
    assert e.value.status == -4


def test_gemm_side_stream(orc):
    X, W = synth.gemm_inputs(300, 200, 100, "f32", seed=5)
    ref, bound = orc.gemm_nt(X, W, "f32")
    s = torch.cuda.Stream()
    x, w = to_device(X, "f32"), to_device(W, "f32")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        case("gemm on a side stream")
        y = cas.gemm_nt(x, w)
    s.synchronize()
    assert_close(y.cpu().numpy(), ref, bound, "f32", "gemm side stream")


# ------------------------------------------------------------ trimul_causal

def run_trimul(qkv, dtype, B, T, NH, HS, label):
    n = B * NH * T * T
    buf, flat = guarded_output(n)
    case(f"{label} trimul_causal {dtype} B={B} T={T} NH={NH} HS={HS}")
    cas.trimul_causal(to_device(qkv, dtype).view(B, T, 3 * NH * HS), NH, out=flat.view(B, NH, T, T))
    torch.cuda.synchronize()
    check_guards(buf, n)
    return flat.view(B, NH, T, T).cpu().numpy()


def run_trimul16(qkv, dtype, out_dtype, B, T, NH, HS, label, offset=0):
    """16-bit score output; offset (elements) shifts the output off 16-byte
    alignment to take the per-element store path."""
    n = B * NH * T * T
    buf, flat = guarded_output16(n + offset, out_dtype)
    out = flat[offset:offset + n].view(B, NH, T, T)
    case(f"{label} trimul_causal {dtype}->{out_dtype} B={B} T={T} NH={NH} HS={HS} offset={offset}")
    cas.trimul_causal(to_device(qkv, dtype).view(B, T, 3 * NH * HS), NH, out=out)
    torch.cuda.synchronize()
    check_guards(buf, n + offset)
    h = flat.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(h[:offset] == 0xFFFF), "wrote before the (shifted) output"
    return h[offset:].reshape(B, NH, T, T)


TRI_T = [1, 2, 7, 63, 64, 65, 127, 128, 129, 300]
TRI_HS = [1, 8, 40, 64, 80, 128]


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("HS", TRI_HS)
@pytest.mark.parametrize("T", TRI_T)
def test_trimul_ragged_f32(orc, monkeypatch, T, HS, kernel):
    """Both score kernels: the super-tile kernel (used where rows are 16-byte
    aligned and the head is at most 256 bytes; other shapes fall back) and the
    per-wave tile kernel that serves every shape."""
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    for (B, NH) in [(1, 1), (2, 3)]:
        qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=T * 131 + HS)
        ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32")
        out = run_trimul(qkv, "f32", B, T, NH, HS, "sweep")
        assert_scores(out, ref, bound, "f32", f"trimul f32 B={B} T={T} NH={NH} HS={HS}")


@pytest.mark.parametrize("passw", ["1", "2", "4"])
@pytest.mark.parametrize("dtype,HS", [("f32", 16), ("f32", 64), ("f32", 72), ("bf16", 32), ("bf16", 136), ("f16", 24)])
def test_trimul_tile_pass_widths(orc, monkeypatch, dtype, HS, passw):
    """The tile kernel's register pass width (CAS_TRIMUL_PASS, tuning): every
    width against every head size, one pass or several, including the width
    the automatic choice takes only for 33..64-byte heads."""
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", "tile")
    monkeypatch.setenv("CAS_TRIMUL_PASS", passw)
    for T in (65, 300):
        B, NH = 2, 3
        qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 13 + HS)
        ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
        out = run_trimul(qkv, dtype, B, T, NH, HS, f"pass {passw}")
        assert_scores(out, ref, bound, dtype, f"trimul tile pass {passw} {dtype} T={T} HS={HS}")


@pytest.mark.parametrize("HS", [40, 64])
@pytest.mark.parametrize("T", [897, 1153])
def test_trimul_item_runs_f32(orc, T, HS):
    """fp32 inputs with eight or more 128-row blocks (T > 896): each workgroup
    walks one contiguous run of items and keeps the Q rows in LDS across
    consecutive items of a triangle row. 32 planes give runs of four or five
    items that start and end mid-row; every element against the oracle."""
    B, NH = 4, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=T * 17 + HS)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32")
    out = run_trimul(qkv, "f32", B, T, NH, HS, "item runs")
    assert_scores(out, ref, bound, "f32", f"trimul item runs f32 B={B} T={T} NH={NH} HS={HS}")


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("HS", [8, 40, 64, 80, 128, 136, 3])
@pytest.mark.parametrize("T", [1, 65, 128, 300])
def test_trimul_ragged_16bit(orc, monkeypatch, T, HS, dtype, kernel):
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 17 + HS)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul(qkv, dtype, B, T, NH, HS, "sweep16")
    assert_scores(out, ref, bound, dtype, f"trimul {dtype} T={T} HS={HS}")


WIDE_HEADS = [("f32", 68), ("f32", 96), ("f32", 100), ("f32", 112), ("f32", 128), ("bf16", 136), ("bf16", 200), ("bf16", 256), ("f16", 144)]


@pytest.mark.parametrize("T", [1, 65, 128, 129, 300])
@pytest.mark.parametrize("dtype,HS", WIDE_HEADS, ids=lambda v: str(v))
def test_trimul_wide_heads_two_halves(orc, monkeypatch, T, dtype, HS):
    """Heads of 257 .. 512 bytes (the second half whole or partial): the
    super-tile kernel in two head halves against the oracle, and bit for bit
    against the per-wave tile kernel, which forms the same products in the
    same order."""
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 71 + HS)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul(qkv, dtype, B, T, NH, HS, "two halves")
    assert_scores(out, ref, bound, dtype, f"trimul two halves {dtype} T={T} HS={HS}")
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", "tile")
    out_t = run_trimul(qkv, dtype, B, T, NH, HS, "two halves, tile kernel")
    assert np.array_equal(out.view(np.uint32), out_t.view(np.uint32)), "super-tile and tile kernels differ"


@pytest.mark.parametrize("dtype,HS", [("f32", 128), ("f32", 80), ("bf16", 256), ("bf16", 136)], ids=lambda v: str(v))
def test_trimul_wide_heads_many_items(orc, monkeypatch, dtype, HS):
    """Two head halves over many super-tiles per workgroup (B2 T1024 NH8:
    576 items on a grid of at most one workgroup per CU), so every
    workgroup walks several items (operand halves, mirror and output buffer
    handed on from item to item): the whole output against the oracle, and
    bit for bit against the tile kernel."""
    B, T, NH = 2, 1024, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 81)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul(qkv, dtype, B, T, NH, HS, "two halves many items")
    assert_scores(out, ref, bound, dtype, f"trimul two halves many items {dtype} HS={HS}")
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", "tile")
    out_t = run_trimul(qkv, dtype, B, T, NH, HS, "two halves many items, tile kernel")
    assert np.array_equal(out.view(np.uint32), out_t.view(np.uint32)), "super-tile and tile kernels differ"


# Heads that end inside a 16-byte piece (fp32 HS not a multiple of 4, 16-bit
# HS not a multiple of 8), up to 512 bytes: the super-tile kernel with the
# last piece's bytes past the head zeroed in registers (one and two head
# halves), against the oracle and bit for bit against the tile kernel's
# element-wise fetch.
PART_HEADS = [("f32", 1), ("f32", 3), ("f32", 50), ("f32", 66), ("f32", 127), ("bf16", 3), ("bf16", 36),
              ("bf16", 100), ("bf16", 129), ("bf16", 190), ("f16", 12), ("f16", 250)]


@pytest.mark.parametrize("T", [1, 65, 300])
@pytest.mark.parametrize("dtype,HS", PART_HEADS, ids=lambda v: str(v))
def test_trimul_partial_piece_heads(orc, monkeypatch, T, dtype, HS):
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 89 + HS)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul(qkv, dtype, B, T, NH, HS, "partial piece")
    assert_scores(out, ref, bound, dtype, f"trimul partial piece {dtype} T={T} HS={HS}")
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", "tile")
    out_t = run_trimul(qkv, dtype, B, T, NH, HS, "partial piece, tile kernel")
    assert np.array_equal(out.view(np.uint32), out_t.view(np.uint32)), "super-tile and tile kernels differ"


@pytest.mark.parametrize("dtype,HS", [("f32", 66), ("bf16", 100)], ids=lambda v: str(v))
def test_trimul_partial_piece_many_items_and_out16(orc, dtype, HS):
    """Partial-piece heads over many super-tiles per workgroup (B2 T1024 NH8),
    the whole output against the oracle, and bf16 output."""
    B, T, NH = 2, 1024, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 91)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul(qkv, dtype, B, T, NH, HS, "partial piece many items")
    assert_scores(out, ref, bound, dtype, f"trimul partial piece many items {dtype} HS={HS}")
    q2 = synth.trimul_inputs(2, 300, 2, HS, dtype, seed=HS + 93)
    ref2, bound2 = orc.trimul_causal(q2, 2, 300, 2 * HS, 2, dtype)
    out16 = run_trimul16(q2, dtype, "bf16", 2, 300, 2, HS, "partial piece out16")
    assert_scores16(out16, ref2, bound2, dtype, "bf16", f"trimul partial piece {dtype}->bf16 HS={HS}")


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype,HS", [("f32", 100), ("bf16", 256)], ids=lambda v: str(v))
def test_trimul_wide_heads_out16(orc, dtype, HS, out_dtype):
    for T in (200, 257):
        B, NH = 2, 2
        qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 73 + HS)
        ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
        out = run_trimul16(qkv, dtype, out_dtype, B, T, NH, HS, "two halves out16")
        assert_scores16(out, ref, bound, dtype, out_dtype, f"trimul two halves {dtype}->{out_dtype} T={T} HS={HS}")


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_trimul_exact_small_integers(orc, monkeypatch, dtype, kernel):
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    for (B, T, NH, HS) in [(2, 257, 2, 64), (1, 130, 3, 40)]:
        qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS, dist="int")
        ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
        out = run_trimul(qkv, dtype, B, T, NH, HS, "exact")
        # HS = 64 scales by 1/8 exactly; HS = 40 rounds once, like the oracle
        assert_scores(out, ref, bound, dtype, f"trimul exact {dtype}", exact=(HS == 64))


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("HS", [40, 64])
@pytest.mark.parametrize("T", [1, 65, 128, 200, 256])
def test_trimul_out16(orc, monkeypatch, T, HS, dtype, out_dtype, kernel):
    """16-bit score output: whole and ragged tiles, rows 16-byte aligned
    (T % 8 == 0) or not, both kernels."""
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 29 + HS)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul16(qkv, dtype, out_dtype, B, T, NH, HS, "out16")
    assert_scores16(out, ref, bound, dtype, out_dtype, f"trimul {dtype}->{out_dtype} T={T} HS={HS}")


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_trimul_out16_exact(orc, monkeypatch, dtype, out_dtype, kernel):
    """Integer inputs and HS = 64 (scale 1/8): the fp32 scores are exact, so
    the 16-bit outputs must equal the oracle's rounding of them bit for bit."""
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    B, T, NH, HS = 2, 257, 2, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 1, dist="int")
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    out = run_trimul16(qkv, dtype, out_dtype, B, T, NH, HS, "out16 exact")
    assert_scores16(out, ref, bound, dtype, out_dtype, f"trimul exact {dtype}->{out_dtype}",
                    exact16=orc.round16(ref, out_dtype))


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_trimul_out16_unaligned(orc, monkeypatch, out_dtype, kernel):
    """Output one element past a 16-byte boundary: the per-element stores."""
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    B, T, NH, HS = 2, 136, 2, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", seed=77)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, "bf16")
    out = run_trimul16(qkv, "bf16", out_dtype, B, T, NH, HS, "out16 unaligned", offset=1)
    assert_scores16(out, ref, bound, "bf16", out_dtype, f"trimul unaligned ->{out_dtype}")


@pytest.mark.parametrize("kernel", ["super", "tile"])
@pytest.mark.parametrize("HS", [16, 64, 128])
@pytest.mark.parametrize("offset", [1, 3])
@pytest.mark.parametrize("dtype", DTYPES)
def test_trimul_misaligned_base(orc, monkeypatch, dtype, offset, HS, kernel):
    """qkv `offset` elements past a 16-byte boundary: the 16-byte pieces are
    loaded at the base's offset within a line. Against the oracle, and bit for
    bit against the same input at an aligned base."""
    monkeypatch.setenv("CAS_TRIMUL_KERNEL", kernel)
    B, T, NH = 2, 70, 2
    n = B * T * 3 * NH * HS
    flat = synth.to_storage(synth.normal_f32(synth.rng(3 + HS), (n + offset,)), dtype)
    qkv = flat[offset:].reshape(B, T, 3 * NH * HS)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, dtype)
    d = to_device(flat, dtype)
    buf, o = guarded_output(B * NH * T * T)
    case(f"trimul misaligned {dtype} offset={offset} HS={HS} {kernel}")
    cas.trimul_causal(d[offset:].view(B, T, -1), NH, out=o.view(B, NH, T, T))
    torch.cuda.synchronize()
    check_guards(buf, B * NH * T * T)
    got = o.view(B, NH, T, T).cpu().numpy()
    assert_scores(got, ref, bound, dtype, f"trimul misaligned {dtype} offset={offset} HS={HS}")
    aligned = run_trimul(qkv, dtype, B, T, NH, HS, "aligned twin")
    assert np.array_equal(got.view(np.uint32), aligned.view(np.uint32)), "misaligned base changes the scores"


def test_trimul_5d_input_and_side_stream(orc):
    B, T, NH, HS = 1, 200, 4, 32
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", seed=8)
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, "bf16")
    d = to_device(qkv, "bf16").view(B, T, 3, NH, HS)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        case("trimul 5-d input on a side stream")
        out = cas.trimul_causal(d, NH)
    s.synchronize()
    assert_scores(out.cpu().numpy(), ref, bound, "bf16", "trimul 5d")


def test_trimul_alias_rejected():
    buf = torch.zeros(1 << 16, device="cuda")
    qkv = buf[:2 * 8 * 24].view(2, 8, 24)
    with pytest.raises(cas.CasError) as e:
        cas.trimul_causal(qkv, 2, out=buf[100:100 + 2 * 2 * 64].view(2, 2, 8, 8))
    assert e.value.status == -4


def test_trimul_rejects_bad_heads():
    qkv = torch.zeros((1, 4, 30), device="cuda")
    with pytest.raises(cas.CasError):
        cas.trimul_causal(qkv, 4)  # C = 10 is not a multiple of NH = 4


# ------------------------------------------------- the five workloads, full size

def test_workload_dense_f32_15x9x12(orc):
    wl = synth.WORKLOADS["dense_f32_15x9x12"]
    X, W = wl.inputs()
    ref, bound = orc.gemm_nt(X, W, "f32")
    y = run_gemm(X, W, "f32", 15, 9, 12, wl.name)
    assert_close(y, ref, bound, "f32", wl.name)
    # the same product taken the notebook's tiled way
    tiled, loads, writes, _, _ = orc.tiled_matmul_count(X, np.ascontiguousarray(W.T), 5, 3, 6)
    assert (loads, writes) == (864, 135)
    assert np.max(np.abs(y - tiled)) <= 1e-4 * np.max(bound) + 1e-6


def test_workload_dense_f32_960x1024x770(orc):
    wl = synth.WORKLOADS["dense_f32_960x1024x770"]
    X, W = wl.inputs()
    ref, bound = orc.gemm_nt(X, W, "f32")
    y = run_gemm(X, W, "f32", 960, 1024, 770, wl.name)
    r = assert_close(y, ref, bound, "f32", wl.name)
    print(f"{wl.name}: max err/tol {r:.3g}")


@pytest.mark.parametrize("variant", ["local_padding", "predicated"])
def test_workload_dense_f32_960x2304x770(orc, monkeypatch, variant):
    """The local-padding A/B shape, both variants, in the launch configuration
    bench.py times (automatic tile choice)."""
    if variant == "predicated":
        monkeypatch.setenv("CAS_VARIANT", "predicated")
    wl = synth.WORKLOADS["dense_f32_960x2304x770"]
    M, N, K = wl.dims
    X, W = wl.inputs()
    ref, bound = orc.gemm_nt(X, W, "f32")
    y = run_gemm(X, W, "f32", M, N, K, f"{wl.name} {variant}")
    r = assert_close(y, ref, bound, "f32", f"{wl.name} {variant}")
    print(f"{wl.name} {variant}: max err/tol {r:.3g}")


@pytest.mark.parametrize("variant", ["local_padding", "predicated"])
def test_workload_bmm_nt_f32_192x120x120x64(orc, monkeypatch, variant):
    """DietCode's BatchMatmulNT heads, whole output, both variants, in the
    launch configuration bench.py times."""
    if variant == "predicated":
        monkeypatch.setenv("CAS_VARIANT", "predicated")
    wl = synth.WORKLOADS["bmm_nt_f32_192x120x120x64"]
    X, W = wl.inputs()
    ref, bound = orc.batch_matmul_nt(X, W, "f32")
    y = run_bmm(X, W, "f32", f"{wl.name} {variant}")
    r = assert_close(y, ref, bound, "f32", f"{wl.name} {variant}")
    print(f"{wl.name} {variant}: max err/tol {r:.3g}")


def test_workload_trimul_f32_B16_T120(orc):
    """Ragged-T causal scores of the same heads, from packed QKV, whole output."""
    wl = synth.WORKLOADS["trimul_f32_B16_T120_NH12_HS64"]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    ref, bound = orc.trimul_causal(qkv, B, T, NH * HS, NH, "f32")
    case(f"{wl.name} full size")
    out = cas.trimul_causal(to_device(qkv, "f32").view(B, T, 3 * NH * HS), NH)
    torch.cuda.synchronize()
    assert_scores(out.cpu().numpy(), ref, bound, "f32", wl.name)


def test_workload_trimul_f32_B8_T1024(orc):
    wl = synth.WORKLOADS["trimul_f32_B8_T1024_NH12_HS64"]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    out = run_trimul(qkv, "f32", B, T, NH, HS, wl.name)
    worst = 0.0
    for b in range(B):
        for h in range(NH):
            ref, bound = orc.trimul_causal_rows(qkv, B, T, NH * HS, NH, b, h, 0, T, "f32")
            worst = max(worst, assert_scores(out[b, h], ref, bound, "f32", f"{wl.name} plane ({b},{h})"))
    print(f"{wl.name}: max err/tol {worst:.3g}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["dense_bf16_4096", "dense_f16_4096"])
def test_workload_dense_4096_whole(orc, name):
    """M = N = K = 4096 with 16-bit inputs in the launch configuration the
    benchmark times (256 x 256 tiles, one per CU): the output starts as the
    sentinel between guard bands, and every one of its 16.8 M elements is
    compared with the oracle's (all 4096 rows, 256 workgroups)."""
    wl = synth.WORKLOADS[name]
    M, N, K = wl.dims
    X, W = wl.inputs()
    y = run_gemm(X, W, wl.dtype, M, N, K, f"{wl.name} full size")
    ref, bound = orc.gemm_nt(X, W, wl.dtype)
    r = assert_close(y, ref, bound, wl.dtype, wl.name)
    print(f"{wl.name}: every element, max err/tol {r:.3g}")


def _plane_oracle(orc, qkv, wl):
    """Oracle planes (b, nh) in order, each computed on a worker thread while
    the previous one is compared (the oracle releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    B, T, NH, HS = wl.dims
    P = B * NH
    with ThreadPoolExecutor(1) as ex:
        fut = ex.submit(orc.trimul_causal_rows, qkv, B, T, NH * HS, NH, 0, 0, 0, T, wl.dtype)
        for p in range(P):
            ref, bound = fut.result()
            if p + 1 < P:
                b1, h1 = divmod(p + 1, NH)
                fut = ex.submit(orc.trimul_causal_rows, qkv, B, T, NH * HS, NH, b1, h1, 0, T, wl.dtype)
            yield divmod(p, NH), ref, bound


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,out16", [("trimul_bf16_B4_T4096_NH25_HS64", "bf16"),
                                        ("trimul_f16_B4_T4096_NH25_HS64", "f16")])
def test_workload_trimul_B4_T4096_whole(orc, name, out16):
    """The large score shape, QKV (4, 4096, 3, 25, 64) with 16-bit inputs,
    in the launch configuration the benchmark times, into an fp32 output
    (the bf16 case is the fp32-output workload of the contract) and into a
    16-bit one. Both outputs start as the sentinel between guard bands; every
    element of all 100 (T, T) planes of both is compared with the oracle's
    plane: the NaN pattern exactly above the diagonal, the tolerance on and
    below it."""
    wl = synth.WORKLOADS[name]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    d = to_device(qkv, wl.dtype)
    n = B * NH * T * T
    buf32, flat32 = guarded_output(n)
    buf16, flat16 = guarded_output16(n, out16)
    o32, o16 = flat32.view(B, NH, T, T), flat16.view(B, NH, T, T)
    case(f"{wl.name} -> f32 trimul_causal full size")
    cas.trimul_causal(d, NH, out=o32)
    torch.cuda.synchronize()
    case(f"{wl.name} -> {out16} trimul_causal full size")
    cas.trimul_causal(d, NH, out=o16)
    torch.cuda.synchronize()
    check_guards(buf32, n)
    check_guards(buf16, n)
    up = upper_mask(T)
    w32 = w16 = 0.0
    for (b, h), ref, bound in _plane_oracle(orc, qkv, wl):
        if (b * NH + h) % 10 == 0:
            case(f"{wl.name}: comparing plane ({b},{h}) of {B * NH}")
        w32 = max(w32, assert_plane_scores(o32[b, h].cpu().numpy(), ref, bound, wl.dtype,
                                           f"{wl.name} -> f32 plane ({b},{h})", up))
        g16 = o16[b, h].view(torch.int16).cpu().numpy().view(np.uint16)
        w16 = max(w16, assert_plane_scores16(g16, ref, bound, wl.dtype, out16,
                                             f"{wl.name} -> {out16} plane ({b},{h})", up))
    print(f"{wl.name}: every element of all {B * NH} planes, max err/tol {w32:.3g} (f32 out), "
          f"{w16:.3g} ({out16} out)")
