"""GPU parity of the causal softmax (cas_causal_row_stats, cas_causal_softmax)
against the CPU oracle, through the C ABI.

The tolerance is derived from the score tolerance (see gpu_util): max and
log-sum-exp are 1-Lipschitz in the largest score error, plus fp32 summation
and rounding terms. Inputs whose scores are exact in fp32 (the ramp rows)
leave only the latter, a tight check of the GPU's exp / log / sum arithmetic.
Masked entries must be the fill pattern bit for bit."""
import numpy as np
import pytest
import torch

import causal_attention_score_amd as cas
from causal_attention_score_amd import synth
from gpu_util import (FILL, GUARD, ROUND16, SENTINEL, SENTINEL16, SM_R, assert_attention, assert_attention_online,
                      assert_softmax, assert_softmax_stats, case, check_guards, online_logsum_extra,
                      guarded_output, guarded_output16, softmax_allowance, to_device)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "f16"]


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


LAUNCHES = ["two", "fused"]


def device_qkv(qkv, dtype, B, T, NH, HS, offset=0):
    """qkv on the device as a contiguous (B, T, 3C) tensor whose base lies
    `offset` elements past an allocation's start (offset 1: a base that is
    not 16-byte aligned)."""
    d = to_device(qkv, dtype).reshape(-1)
    if offset:
        buf = torch.zeros(d.numel() + offset, dtype=d.dtype, device="cuda")
        buf[offset:] = d
        d = buf[offset:]
    return d.view(B, T, 3 * NH * HS)


def run_softmax(qkv, dtype, B, T, NH, HS, mode, out_dtype="f32", label="", offset=0, launch="two", qkv_offset=0):
    """The softmax into guarded buffers, as two launches (row statistics, then
    softmax rows) or the fused one; returns (out rows (B*NH*T, T) as float32
    or raw uint16, row_max (B*NH*T,), row_logsum (B*NH*T,))."""
    d = device_qkv(qkv, dtype, B, T, NH, HS, qkv_offset)
    ns = B * NH * T
    bm, mx = guarded_output(ns)
    bl, ls = guarded_output(ns)
    n = B * NH * T * T
    if out_dtype == "f32":
        buf, flat = guarded_output(n + offset)
    else:
        buf, flat = guarded_output16(n + offset, out_dtype)
    out = flat[offset:offset + n].view(B, NH, T, T)
    if launch == "fused":
        case(f"{label} causal_softmax_fused {mode} {dtype}->{out_dtype} B={B} T={T} NH={NH} HS={HS} offset={offset}")
        st = cas.lib().cas_causal_softmax_fused(d.data_ptr(), out.data_ptr(), mx.data_ptr(), ls.data_ptr(), B, T,
                                                NH * HS, NH, cas.SOFTMAX_MODE[mode], cas._dtype_code(d),
                                                cas._dtype_code(out), cas._stream_ptr(d.device))
        assert st == 0, cas.status_string(st)
    else:
        case(f"{label} causal_row_stats {dtype} B={B} T={T} NH={NH} HS={HS}")
        cas.causal_row_stats(d, NH, row_max=mx.view(B, NH, T), row_logsum=ls.view(B, NH, T))
        torch.cuda.synchronize()
        case(f"{label} causal_softmax {mode} {dtype}->{out_dtype} B={B} T={T} NH={NH} HS={HS} offset={offset}")
        cas.causal_softmax(d, NH, mode, out=out, stats=(mx.view(B, NH, T), ls.view(B, NH, T)))
    torch.cuda.synchronize()
    check_guards(bm, ns)
    check_guards(bl, ns)
    check_guards(buf, n + offset)
    if out_dtype == "f32":
        h = flat.cpu().numpy()
        assert np.all(h[:offset].view(np.uint32) == 0xFFFFFFFF), "wrote before the (shifted) output"
    else:
        h = flat.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.all(h[:offset] == 0xFFFF), "wrote before the (shifted) output"
    return h[offset:].reshape(ns, T), mx.cpu().numpy().astype(np.float64), ls.cpu().numpy().astype(np.float64)


def oracle_rows(orc, qkv, dtype, B, T, NH, HS, mode):
    out, mx, ls, bound = orc.causal_softmax(qkv, B, T, NH * HS, NH, dtype, mode)
    ns = B * NH * T
    return out.reshape(ns, T), mx.reshape(ns), ls.reshape(ns), bound.reshape(ns, T)


def check_case(orc, qkv, dtype, B, T, NH, HS, mode, out_dtype="f32", label="", offset=0, exact_scores=False,
               launch="two", qkv_offset=0):
    got, mx, ls = run_softmax(qkv, dtype, B, T, NH, HS, mode, out_dtype, f"{label} {launch}", offset, launch,
                              qkv_offset)
    ref, mref, lref, bound = oracle_rows(orc, qkv, dtype, B, T, NH, HS, mode)
    t_idx = np.tile(np.arange(T), B * NH)
    what = f"{label} {mode} {dtype}->{out_dtype} B={B} T={T} NH={NH} HS={HS}"
    q1 = assert_softmax_stats(mx, ls, mref, lref, bound, t_idx, dtype, what, exact_scores)
    q2 = assert_softmax(got, ref, lref, bound, t_idx, dtype, mode, out_dtype, what, exact_scores)
    return max(q1, q2)


SM_T = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300]


@pytest.mark.parametrize("dtype", DTYPES)
def test_softmax_default_launch(dtype):
    """Without stats or fused, the binding takes the two launches for fp32
    inputs and the fused launch for 16-bit inputs: outputs and statistics
    equal those of that explicit choice bit for bit."""
    B, T, NH, HS = 2, 200, 3, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=17)
    d = to_device(qkv, dtype).view(B, T, -1)
    case(f"softmax default launch {dtype}")
    want = dtype != "f32"
    got = cas.causal_softmax(d, NH, "prob")
    ref = cas.causal_softmax(d, NH, "prob", fused=want)
    torch.cuda.synchronize()
    for g, r, name in zip(got, ref, ("probabilities", "row_max", "row_logsum")):
        assert torch.equal(g.view(torch.int32), r.view(torch.int32)), f"{name} differ from fused={want}"


@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("HS", [8, 16, 40, 64])
@pytest.mark.parametrize("T", SM_T)
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_ragged_f32(orc, launch, T, HS, mode):
    for (B, NH) in [(1, 1), (2, 3)]:
        qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=T * 7 + HS)
        check_case(orc, qkv, "f32", B, T, NH, HS, mode, label="sweep", launch=launch)


@pytest.mark.parametrize("mode", ["prob", "log"])
def test_softmax_item_runs_f32(orc, mode):
    """The two-launch rows on fp32 inputs with eight 128-row blocks, where the
    rows kernel walks contiguous item runs and keeps Q rows (and their
    statistics) in LDS across items: 32 planes, every element."""
    B, T, NH, HS = 4, 1000, 8, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=1000 * 7 + HS)
    check_case(orc, qkv, "f32", B, T, NH, HS, mode, label="item runs", launch="two")


@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("HS", [8, 64, 128])
@pytest.mark.parametrize("T", [1, 65, 128, 129, 300])
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_ragged_16bit(orc, launch, T, HS, dtype, mode):
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 11 + HS)
    check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="sweep16", launch=launch)


# The fused launch has two walks for 16-bit inputs with heads of at most 128
# bytes: the plain one (each block's statistics steps, then its output steps)
# and the pipelined one (a block's output steps carry the next block's
# statistics steps), chosen by the number of query blocks. Both are forced
# here on ragged shapes, checked against the oracle and against each other:
# they must agree bit for bit, statistics and every output byte included.
PIPE_SHAPES = [(1, 1, 1, 64), (2, 65, 3, 64), (1, 300, 2, 40), (3, 1100, 2, 16), (2, 2049, 1, 64)]


@pytest.mark.parametrize("walk", ["pipe", "split"])
@pytest.mark.parametrize("out_dtype", ["same", "f32"])
@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", PIPE_SHAPES, ids=lambda s: "B%dT%dNH%dHS%d" % s)
def test_softmax_fused_pipelined_walk(orc, monkeypatch, shape, dtype, mode, out_dtype, walk):
    """The pipelined walk (statistics of the next query block beside the
    outputs of the current one), in the compute waves themselves ("pipe") or
    on waves of their own ("split"): against the oracle, and bit for bit
    against the plain walk."""
    B, T, NH, HS = shape
    od = dtype if out_dtype == "same" else out_dtype
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 13 + HS)
    monkeypatch.setenv("CAS_SOFTMAX_FUSED", walk)
    check_case(orc, qkv, dtype, B, T, NH, HS, mode, od, label=f"{walk} walk", launch="fused")
    got_p = run_softmax(qkv, dtype, B, T, NH, HS, mode, od, f"{walk} walk", launch="fused")
    monkeypatch.setenv("CAS_SOFTMAX_FUSED", "plain")
    got_q = run_softmax(qkv, dtype, B, T, NH, HS, mode, od, "plain walk", launch="fused")
    for a, b in zip(got_p, got_q):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), f"walks differ at {shape}"


@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_ramp_rows_exact_scores(orc, launch, dtype, mode):
    """Ramp score rows slope * t2 (exact in fp32 for every input type): only
    the fp32 exp / log / sum error is allowed. Slopes 0.25, -0.5, 0 and 64
    (saturated: row maxima up to 64 * 299)."""
    B, T, NH, HS = 2, 300, 4, 64
    slopes = [0.25, -0.5, 0.0, 64.0]
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in slopes], dtype)
    check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="ramp", exact_scores=True, launch=launch)


@pytest.mark.parametrize("dtype", DTYPES)
def test_softmax_stats_match_the_score_kernel(orc, dtype):
    """The recomputed scores are the score kernel's, bit for bit: row_max is
    the largest fp32 score of cas_trimul_causal's row, and the largest
    log-probability of a row is exactly -row_logsum."""
    B, T, NH, HS = 2, 333, 3, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=91)
    d = to_device(qkv, dtype).view(B, T, -1)
    case(f"stats vs scores {dtype}")
    sc = cas.trimul_causal(d, NH)
    low = torch.tril(torch.ones(T, T, dtype=torch.bool, device="cuda"))
    smax = torch.where(low, sc, torch.full_like(sc, -float("inf"))).amax(dim=-1)
    res = {}
    for fused in (False, True):
        lp, mx, ls = cas.causal_softmax(d, NH, "log", fused=fused)
        torch.cuda.synchronize()
        assert torch.equal(smax.view(torch.int32), mx.view(torch.int32)), f"row_max (fused={fused})"
        assert torch.equal(lp.amax(dim=-1).view(torch.int32), (-ls).view(torch.int32)), f"max lp (fused={fused})"
        res[fused] = ls
    # the two launches and the fused one sum in different orders: logsums agree to fp32 summation error
    n = torch.arange(1, T + 1, device="cuda", dtype=torch.float32)
    assert bool(((res[False] - res[True]).abs() <= (2 * n + 128) * 2.0 ** -24 + 2.0 ** -20).all())


@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [65, 128, 200, 256])
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_out16(orc, launch, T, dtype, out_dtype, mode):
    B, NH, HS = 2, 3, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 3 + 5)
    check_case(orc, qkv, dtype, B, T, NH, HS, mode, out_dtype, label="out16", launch=launch)


@pytest.mark.parametrize("out_dtype,offset", [("f32", 1), ("bf16", 1), ("f16", 3)])
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_unaligned_output(orc, launch, out_dtype, offset):
    """Output off a 16-byte boundary: the per-element store path."""
    B, T, NH, HS = 2, 136, 2, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", seed=17)
    for mode in ("prob", "log"):
        check_case(orc, qkv, "bf16", B, T, NH, HS, mode, out_dtype, label="unaligned", offset=offset,
                   launch=launch)


@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_saturated(orc, launch):
    """Inputs scaled by 64: scores of order 1e3-1e4 (exp of a score overflows
    fp32). The two statistics stay separate numbers, so nothing overflows.
    Statistics and log-probabilities are compared with their allowances. At
    this scale the score allowance moves a probability by orders of magnitude,
    so the probabilities are checked for what holds whatever the score error:
    finite, the fill exact, and each row summing to one. Their values at this
    scale are compared on exact scores (the slope-64 ramp rows)."""
    B, T, NH, HS = 1, 257, 2, 64
    qkv = (synth.trimul_inputs(B, T, NH, HS, "f32", seed=5) * np.float32(64.0)).astype(np.float32)
    check_case(orc, qkv, "f32", B, T, NH, HS, "log", label="saturated", launch=launch)
    got, mx, ls = run_softmax(qkv, "f32", B, T, NH, HS, "prob", "f32", f"saturated {launch}", 0, launch)
    _, mref, lref, bound = oracle_rows(orc, qkv, "f32", B, T, NH, HS, "prob")
    t_idx = np.tile(np.arange(T), B * NH)
    assert_softmax_stats(mx, ls, mref, lref, bound, t_idx, "f32", "saturated prob")
    valid = np.arange(T)[None, :] <= t_idx[:, None]
    assert np.all(got.view(np.uint32)[~valid] == 0), "fill above the diagonal"
    p = got.astype(np.float64)
    assert np.all(np.isfinite(p)) and np.all(p >= 0)
    # sum_j p_j = 2^(-dL) sum_j exact_j (1 + e_j): the GPU's logsum of its own
    # scores is within S + R (1 + L), each p_j within 2^-24 (2 + 5 |ln p_j|)
    lnp = np.log(np.where(p > 0, p, 1.0))
    n = t_idx + 1
    lim = (n + 64) * 2.0 ** -24 + SM_R * (1 + np.abs(ls)) + (p * 2.0 ** -24 * (2 + 5 * np.abs(lnp))).sum(axis=1)
    err = np.abs(p.sum(axis=1) - 1.0)
    assert np.all(err <= lim), f"row sums: worst {float((err / lim).max()):.3g} of the allowance"


def test_softmax_big_heads_and_rejections():
    """HS = 200 fp32 (800-byte heads, staged in two chunks) is served: zero
    inputs give uniform rows. An fp32 base off its 4-byte alignment is
    rejected, with nothing written."""
    qkv = torch.zeros(2, 8, 3 * 2 * 200, device="cuda")
    for fused in (False, True):
        p, mx, ls = cas.causal_softmax(qkv, 2, fused=fused)
        torch.cuda.synchronize()
        assert torch.equal(mx, torch.zeros_like(mx)), "row maxima of zero scores"
        assert bool((p.sum(-1) - 1).abs().max() < 1e-6), "rows sum to one"
    buf = torch.zeros(2 * 8 * 3 * 2 * 8 + 1, device="cuda")
    mx = torch.full((2, 2, 8), 7.0, device="cuda")
    ls = torch.full((2, 2, 8), 7.0, device="cuda")
    st = cas.lib().cas_causal_row_stats(buf.data_ptr() + 2, mx.data_ptr(), ls.data_ptr(), 2, 8, 16, 2,
                                        cas.CAS_F32, cas._stream_ptr(buf.device))
    assert st == -7
    torch.cuda.synchronize()
    assert bool((mx == 7.0).all()) and bool((ls == 7.0).all()), "a rejected call wrote"
    with pytest.raises(ValueError):
        cas.causal_softmax(torch.zeros(2, 8, 3 * 2 * 8, device="cuda"), 2, mode="softmax")


def test_softmax_output_over_statistics_rejected():
    qkv = torch.zeros(1, 8, 3 * 2 * 8, device="cuda")
    buf = torch.zeros(4096, device="cuda")
    mx, ls = buf[:16].view(1, 2, 8), buf[16:32].view(1, 2, 8)
    cas.causal_row_stats(qkv, 2, row_max=mx, row_logsum=ls)
    with pytest.raises(cas.CasError) as e:
        cas.causal_softmax(qkv, 2, out=buf[:128].view(1, 2, 8, 8), stats=(mx, ls))
    assert e.value.status == -4


def test_softmax_empty_and_side_stream(orc):
    assert cas.causal_softmax(torch.zeros(0, 5, 3 * 8, device="cuda"), 1)[0].numel() == 0
    B, T, NH, HS = 1, 200, 4, 32
    qkv = synth.trimul_inputs(B, T, NH, HS, "bf16", seed=8)
    d = to_device(qkv, "bf16").view(B, T, 3, NH, HS)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        case("softmax 5-d input on a side stream")
        out, mx, ls = cas.causal_softmax(d, NH, "prob")
    s.synchronize()
    ref, mref, lref, bound = oracle_rows(orc, qkv, "bf16", B, T, NH, HS, "prob")
    t_idx = np.tile(np.arange(T), B * NH)
    assert_softmax(out.cpu().numpy().reshape(-1, T), ref, lref, bound, t_idx, "bf16", "prob", "f32", "side stream")


@pytest.mark.parametrize("name,mode,out_dtype,fused", [("trimul_f32_B8_T1024_NH12_HS64", "prob", "f32", True),
                                                       ("trimul_f32_B8_T1024_NH12_HS64", "log", "f32", False),
                                                       ("trimul_bf16_B4_T4096_NH25_HS64", "prob", "bf16", True),
                                                       ("trimul_bf16_B4_T4096_NH25_HS64", "prob", "bf16", False),
                                                       ("trimul_f16_B4_T4096_NH25_HS64", "log", "f16", True)])
def test_workload_softmax_full_size(orc, name, mode, out_dtype, fused):
    """The benchmark's score shapes, in the launch configuration the benchmark
    times. The output starts as the sentinel (a NaN), so the fill above the
    diagonal and finite values on and below it show that every element was
    written. At T = 1024 every plane (statistics and rows) is compared; at
    T = 4096 three whole planes and rows of every seventh plane."""
    wl = synth.WORKLOADS[name]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    d = to_device(qkv, wl.dtype)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out_dtype]
    if out_dtype == "f32":
        out = torch.full((B, NH, T, T), SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)
    else:
        out = torch.full((B, NH, T, T), SENTINEL16, dtype=torch.int16, device="cuda").view(tdt)
    case(f"{wl.name} causal_softmax {mode} -> {out_dtype} full size, fused={fused}")
    _, mx, ls = cas.causal_softmax(d, NH, mode, out=out, fused=fused)
    torch.cuda.synchronize()
    fill = FILL[(out_dtype, mode)]
    iv = out.view(torch.int32) if out_dtype == "f32" else out.view(torch.int16)
    fv = fill if out_dtype == "f32" or fill < 0x8000 else fill - 0x10000
    if out_dtype == "f32" and fill >= 0x80000000:
        fv = fill - 0x100000000
    up = torch.triu(torch.ones(T, T, dtype=torch.bool, device="cuda"), 1)
    n_fill_up = int((iv[..., up] == fv).sum())
    assert n_fill_up == B * NH * T * (T - 1) // 2, "fill above the diagonal"
    assert bool(torch.isfinite(out[..., ~up]).all()), "non-finite value on or below the diagonal"
    del up
    worst = 0.0
    whole = T <= 1024
    planes = [divmod(p, NH) for p in range(B * NH)] if whole else [(0, 0), (B - 1, NH - 1), (B // 2, NH // 3)]
    for (b, h) in planes:
        ref, mref, lref, bound = orc.causal_softmax_rows(qkv, B, T, NH * HS, NH, b, h, 0, T, wl.dtype, mode)
        t_idx = np.arange(T)
        what = f"{wl.name} {mode} plane ({b},{h})"
        worst = max(worst, assert_softmax_stats(mx[b, h].cpu().numpy(), ls[b, h].cpu().numpy(), mref, lref,
                                                bound, t_idx, wl.dtype, what))
        got = out[b, h].cpu().numpy() if out_dtype == "f32" else out[b, h].view(torch.int16).cpu().numpy()
        worst = max(worst, assert_softmax(got, ref, lref, bound, t_idx, wl.dtype, mode, out_dtype, what))
    for p in range(0, 0 if whole else B * NH, 7):
        b, h = divmod(p, NH)
        t0 = (p * 389) % (T - 8)
        ref, mref, lref, bound = orc.causal_softmax_rows(qkv, B, T, NH * HS, NH, b, h, t0, t0 + 8, wl.dtype,
                                                         mode)
        t_idx = np.arange(t0, t0 + 8)
        what = f"{wl.name} {mode} rows {t0}.. plane ({b},{h})"
        worst = max(worst, assert_softmax_stats(mx[b, h, t0:t0 + 8].cpu().numpy(),
                                                ls[b, h, t0:t0 + 8].cpu().numpy(), mref, lref, bound, t_idx,
                                                wl.dtype, what))
        blk = out[b, h, t0:t0 + 8]
        got = blk.cpu().numpy() if out_dtype == "f32" else blk.view(torch.int16).cpu().numpy()
        worst = max(worst, assert_softmax(got, ref, lref, bound, t_idx, wl.dtype, mode, out_dtype, what))
    print(f"{wl.name} softmax {mode} -> {out_dtype} fused={fused}: {'every plane' if whole else 'sampled'} "
          f"max err/tol {worst:.3g}")


# ------------------------------------------------------------ attention output

def run_attention(qkv, dtype, B, T, NH, HS, label, fused_stats=False, qkv_offset=0):
    """Row statistics (two-launch or fused softmax), then the attention output
    into a guarded buffer; returns y (B, T, C)."""
    d = device_qkv(qkv, dtype, B, T, NH, HS, qkv_offset)
    C = NH * HS
    if fused_stats:
        _, mx, ls = cas.causal_softmax(d, NH, "prob", fused=True)
    else:
        mx, ls = cas.causal_row_stats(d, NH)
    n = B * T * C
    buf, flat = guarded_output(n)
    case(f"{label} causal_attention {dtype} B={B} T={T} NH={NH} HS={HS}")
    cas.causal_attention(d, NH, y=flat.view(B, T, C), stats=(mx, ls))
    torch.cuda.synchronize()
    check_guards(buf, n)
    y = flat.view(B, T, C).cpu().numpy()
    assert np.all(np.isfinite(y)), f"{label}: y not written whole (the sentinel is a NaN) or non-finite"
    return y


def check_attention(orc, qkv, dtype, B, T, NH, HS, label, exact_scores=False, fused_stats=False, b_t=None,
                    qkv_offset=0, y=None):
    """GPU attention output against the oracle's, head by head. b_t: optional
    list of (b, t0, t1) row ranges to compare (default: everything). y: an
    output already computed (else the two-pass launches run here)."""
    C = NH * HS
    if y is None:
        y = run_attention(qkv, dtype, B, T, NH, HS, label, fused_stats, qkv_offset)
    V = np.abs(orc.decode(qkv, dtype).reshape(B, T, 3, NH, HS)[:, :, 2]) if dtype != "f32" else \
        np.abs(qkv.reshape(B, T, 3, NH, HS)[:, :, 2].astype(np.float64))
    worst = 0.0
    for (b, t0, t1) in (b_t or [(b, 0, T) for b in range(B)]):
        yr, aw = orc.causal_attention(qkv, B, T, C, NH, dtype, b_range=[b], t_range=(t0, t1))
        for h in range(NH):
            p, _, lr, bd = orc.causal_softmax_rows(qkv, B, T, C, NH, b, h, t0, t1, dtype, "prob")
            cols = slice(h * HS, (h + 1) * HS)
            worst = max(worst, assert_attention(y[b, t0:t1, cols], yr[0, :, cols], aw[0, :, cols], p, lr, bd,
                                                np.arange(t0, t1), V[b, :, h], dtype,
                                                f"{label} attention b={b} h={h} rows {t0}..", exact_scores))
    return worst


@pytest.mark.parametrize("HS", [8, 16, 40, 64])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 300])
def test_attention_ragged_f32(orc, T, HS):
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=T * 13 + HS)
    check_attention(orc, qkv, "f32", B, T, NH, HS, "sweep")


def test_attention_ramp_rows_exact_scores(orc):
    """Ramp scores (exact in fp32) and V entry 0 = key index: y[t][0] is the
    expected key under the row's probabilities (slopes 0.25, -0.5, 0, 64);
    only the fp32 exp / sum error is allowed."""
    B, T, NH, HS = 2, 300, 4, 64
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in (0.25, -0.5, 0.0, 64.0)], "f32", v_ramp=True)
    check_attention(orc, qkv, "f32", B, T, NH, HS, "ramp", exact_scores=True)


# Saturated ramp rows: slopes 64 and 200 per key (row maxima up to 51200) and
# -16, with one gentle slope beside them; exact scores in every input type
# (q0 = 8 * slope is exact in bfloat16 and binary16, keys t2 <= 256 too), and
# random value rows.
SAT_SLOPES = [64.0, -16.0, 0.25, 200.0]


@pytest.mark.parametrize("fused_stats", [False, True])
@pytest.mark.parametrize("dtype", DTYPES)
def test_attention_saturated_ramp(orc, dtype, fused_stats):
    """Saturated rows with exact scores: only the exp / sum roundings (and, for
    16-bit inputs, the rounding of p for the MFMA) are allowed, so every value
    is pinned; statistics from the statistics launch or the fused softmax."""
    B, T, NH, HS = 2, 257, 4, 64
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in SAT_SLOPES], dtype, v_seed=41)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "saturated ramp", exact_scores=True, fused_stats=fused_stats)


def attention_hull_check(orc, y, qkv, dtype, B, T, NH, HS, what):
    """y[t] is a weighted mean of V rows 0..t, whatever the weights: finite and
    inside the per-column range of those rows, up to how far the kernel's
    weights may miss summing to one -- the fp32 sums and roundings of the
    exponentials and the log-sum, 2^-20 (t + 66 + ln(t + 1)), and for 16-bit
    inputs the rounding of each weight to that format for the MFMA."""
    V = orc.decode(qkv, dtype) if dtype != "f32" else np.asarray(qkv, np.float64)
    V = V.reshape(B, T, 3, NH, HS)[:, :, 2]                                     # (B, T, NH, HS)
    lo = np.minimum.accumulate(V, axis=1).reshape(B, T, NH * HS)
    hi = np.maximum.accumulate(V, axis=1).reshape(B, T, NH * HS)
    amax = np.maximum.accumulate(np.abs(V), axis=1).reshape(B, T, NH * HS)
    u16, a16 = ROUND16[dtype] if dtype != "f32" else (0.0, 0.0)
    t = np.arange(T)[None, :, None]
    tol = amax * (u16 + 2.0 ** -20 * (t + 66 + np.log(t + 1.0))) + a16 * (t + 1) * amax
    g = np.asarray(y, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert np.all((g >= lo - tol) & (g <= hi + tol)), f"{what}: output outside the range of the value rows"


@pytest.mark.parametrize("dtype,scale", [("f32", 64.0), ("bf16", 16.0), ("f16", 16.0)])
def test_attention_saturated_random_no_overflow(orc, dtype, scale):
    """Random rows scaled to scores of order 1e2-1e4, where an unshifted
    exponential overflows. The score allowance moves such weights by orders of
    magnitude, so this checks what holds for any weights -- finite outputs
    inside the range of the value rows, for both attention paths -- and the
    row maxima against the oracle's within their allowance; values at this
    scale are compared on exact scores (test_attention_saturated_ramp)."""
    B, T, NH, HS = 1, 257, 2, 64
    qkv = synth.to_storage(synth.trimul_inputs(B, T, NH, HS, "f32", seed=6) * np.float32(scale), dtype)
    y2 = run_attention(qkv, dtype, B, T, NH, HS, "saturated random", fused_stats=True)
    attention_hull_check(orc, y2, qkv, dtype, B, T, NH, HS, f"saturated random {dtype} two-pass")
    y1, mx, _ = run_attention_fused(qkv, dtype, B, T, NH, HS, "saturated random")
    attention_hull_check(orc, y1, qkv, dtype, B, T, NH, HS, f"saturated random {dtype} single pass")
    for h in range(NH):
        _, mref, lref, bd = orc.causal_softmax_rows(qkv, B, T, NH * HS, NH, 0, h, 0, T, dtype, "prob")
        _, D, _, _ = softmax_allowance(bd, np.arange(T), dtype)
        assert np.all(np.abs(mx[0, h] - mref) <= D), f"row maxima, head {h}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("HS", [8, 40, 64, 128])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 129, 300])
def test_attention_ragged_16bit(orc, T, HS, dtype):
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 7 + HS)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "sweep")


def test_attention_rejections():
    # 672-byte binary16 heads are served (staged in chunks): zero values give zero y
    qkv = torch.zeros(2, 8, 3 * 2 * 336, device="cuda", dtype=torch.float16)
    mx = torch.zeros(2, 2, 8, device="cuda")
    y0, _, _ = cas.causal_attention(qkv, 2, stats=(mx, mx))
    torch.cuda.synchronize()
    assert bool((y0 == 0).all())
    # an fp32 base that is not 4-byte aligned (raw pointer through the C ABI)
    buf = torch.zeros(2 * 8 * 3 * 2 * 8 + 1, device="cuda")
    y = torch.zeros(2, 8, 16, device="cuda")
    st = cas.lib().cas_causal_attention(buf.data_ptr() + 2, mx.data_ptr(), mx.data_ptr(), y.data_ptr(), 2, 8, 16, 2,
                                        cas.CAS_F32, cas.CAS_F32, cas._stream_ptr(buf.device))
    assert st == -7


def test_workload_attention_full_size(orc):
    """The fp32 score shape B=8 T=1024 NH=12 HS=64: three whole batches' rows
    of every head compared at sampled ranges."""
    wl = synth.WORKLOADS["trimul_f32_B8_T1024_NH12_HS64"]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    worst = check_attention(orc, qkv, "f32", B, T, NH, HS, wl.name,
                            b_t=[(0, 0, 64), (3, 500, 540), (7, 960, 1024)])
    print(f"{wl.name} attention: sampled max err/tol {worst:.3g}")


def test_workload_attention_bf16_full_size(orc):
    """The bf16 score shape B=4 T=4096: sampled row ranges of every head."""
    wl = synth.WORKLOADS["trimul_bf16_B4_T4096_NH25_HS64"]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    worst = check_attention(orc, qkv, wl.dtype, B, T, NH, HS, wl.name,
                            b_t=[(0, 0, 32), (2, 2040, 2060), (3, 4070, 4096)])
    print(f"{wl.name} attention: sampled max err/tol {worst:.3g}")


# ------------------------------------------------------- single-pass attention

def run_attention_fused(qkv, dtype, B, T, NH, HS, label, y_offset=0, qkv_offset=0):
    """The single-pass attention into guarded buffers (y shifted by y_offset
    elements: 4 gives a y that is only 4-byte aligned); returns y (B, T, C)
    and the statistics (B, NH, T), as numpy."""
    d = device_qkv(qkv, dtype, B, T, NH, HS, qkv_offset)
    C = NH * HS
    n = B * T * C
    ybuf, yflat = guarded_output(n + y_offset)
    y = yflat[y_offset:y_offset + n]
    mbuf, mflat = guarded_output(B * NH * T)
    lbuf, lflat = guarded_output(B * NH * T)
    case(f"{label} causal_attention_fused {dtype} B={B} T={T} NH={NH} HS={HS} y_offset={y_offset}")
    L = cas.lib()
    st = L.cas_causal_attention_fused(d.data_ptr(), y.data_ptr(), mflat.data_ptr(), lflat.data_ptr(), B, T, C, NH,
                                      cas._dtype_code(d), cas.CAS_F32, cas._stream_ptr(d.device))
    cas._check("cas_causal_attention_fused", st)
    torch.cuda.synchronize()
    check_guards(ybuf, n + y_offset)
    check_guards(mbuf, B * NH * T)
    check_guards(lbuf, B * NH * T)
    res = (y.view(B, T, C).cpu().numpy(), mflat.view(B, NH, T).cpu().numpy(), lflat.view(B, NH, T).cpu().numpy())
    for a, name in zip(res, ("y", "row_max", "row_logsum")):
        assert np.all(np.isfinite(a)), f"{label}: {name} not written whole (the sentinel is a NaN) or non-finite"
    return res


def check_attention_fused(orc, qkv, dtype, B, T, NH, HS, label, exact_scores=False, b_t=None, y_offset=0,
                          two_pass_max=True):
    """Single-pass y and statistics against the oracle's, head by head; the
    row maxima also against the two-pass statistics launch, bit for bit."""
    C = NH * HS
    y, mx, ls = run_attention_fused(qkv, dtype, B, T, NH, HS, label, y_offset)
    if two_pass_max:
        mx2, _ = cas.causal_row_stats(to_device(qkv, dtype).view(B, T, 3 * C), NH)
        mx2 = mx2.cpu().numpy()
        if not np.array_equal(mx.view(np.uint32), mx2.view(np.uint32)):
            raise AssertionError(f"{label}: single-pass row_max differs from the statistics launch")
    V = np.abs(orc.decode(qkv, dtype).reshape(B, T, 3, NH, HS)[:, :, 2]) if dtype != "f32" else \
        np.abs(qkv.reshape(B, T, 3, NH, HS)[:, :, 2].astype(np.float64))
    worst = 0.0
    for (b, t0, t1) in (b_t or [(b, 0, T) for b in range(B)]):
        yr, aw = orc.causal_attention(qkv, B, T, C, NH, dtype, b_range=[b], t_range=(t0, t1))
        for h in range(NH):
            p, mr, lr, bd = orc.causal_softmax_rows(qkv, B, T, C, NH, b, h, t0, t1, dtype, "prob")
            cols = slice(h * HS, (h + 1) * HS)
            rows = np.arange(t0, t1)
            what = f"{label} fused attention b={b} h={h} rows {t0}.."
            worst = max(worst, assert_attention_online(y[b, t0:t1, cols], yr[0, :, cols], aw[0, :, cols], p, lr, bd,
                                                       rows, V[b, :, h], dtype, what, exact_scores))
            worst = max(worst, assert_softmax_stats(mx[b, h, t0:t1], ls[b, h, t0:t1], mr, lr, bd, rows, dtype,
                                                    what + " stats", exact_scores, online_logsum_extra(rows)))
    return worst


@pytest.mark.parametrize("HS", [8, 40, 64])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 255, 300])
def test_attention_fused_ragged_f32(orc, T, HS):
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=T * 17 + HS)
    check_attention_fused(orc, qkv, "f32", B, T, NH, HS, "sweep")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("HS", [8, 64, 128])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 129, 300])
def test_attention_fused_ragged_16bit(orc, T, HS, dtype):
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 11 + HS)
    check_attention_fused(orc, qkv, dtype, B, T, NH, HS, "sweep")


def test_attention_fused_ramp_rescales(orc):
    """Ramp scores (exact in fp32) with slopes 0.25, -0.5, 0 and 64 per key:
    the running maximum grows on every step in the steep rows, so the offset
    moves and y is rescaled again and again; only exp / sum roundings allowed."""
    B, T, NH, HS = 2, 300, 4, 64
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in (0.25, -0.5, 0.0, 64.0)], "f32", v_ramp=True)
    check_attention_fused(orc, qkv, "f32", B, T, NH, HS, "ramp", exact_scores=True)


@pytest.mark.parametrize("dtype", DTYPES)
def test_attention_fused_saturated_ramp(orc, dtype):
    """Saturated rows with exact scores in every input type (slopes 64, -16,
    0.25 and 200 per key, random value rows): the offset moves on every step
    of the steep rows and each weight is checked for value, including the
    16-bit rounding of the weights for the MFMA."""
    B, T, NH, HS = 2, 257, 4, 64
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in SAT_SLOPES], dtype, v_seed=43)
    check_attention_fused(orc, qkv, dtype, B, T, NH, HS, "saturated ramp", exact_scores=True)


def test_attention_fused_saturated(orc):
    """Random rows scaled by 16 (scores of order 1e2-1e3) in fp32, where the
    score allowance still pins each weight to within a factor below 1.5."""
    B, T, NH, HS = 1, 257, 2, 64
    qkv = (synth.trimul_inputs(B, T, NH, HS, "f32", seed=6) * np.float32(16.0)).astype(np.float32)
    check_attention_fused(orc, qkv, "f32", B, T, NH, HS, "saturated")


def test_attention_fused_unaligned_y(orc):
    B, T, NH, HS = 2, 70, 3, 16
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=3)
    check_attention_fused(orc, qkv, "f32", B, T, NH, HS, "y+4B", y_offset=1)


def test_attention_fused_empty_and_rejections():
    qkv = torch.zeros(2, 0, 3 * 2 * 8, device="cuda")
    y, mx, ls = cas.causal_attention_fused(qkv, 2)
    assert y.numel() == 0 and mx.numel() == 0
    y2, _, _ = cas.causal_attention(qkv, 2)
    assert y2.numel() == 0
    big = torch.zeros(2, 8, 3 * 2 * 336, device="cuda", dtype=torch.float16)  # 672-byte heads: served
    yb, mxb, _ = cas.causal_attention_fused(big, 2)
    torch.cuda.synchronize()
    assert bool((yb == 0).all()) and bool((mxb == 0).all())
    buf = torch.zeros(2 * 8 * 3 * 2 * 8 + 1, device="cuda")  # an fp32 base off its 4-byte alignment
    y = torch.zeros(2, 8, 16, device="cuda")
    m2, l2 = torch.zeros(2, 2, 8, device="cuda"), torch.zeros(2, 2, 8, device="cuda")
    st = cas.lib().cas_causal_attention_fused(buf.data_ptr() + 2, y.data_ptr(), m2.data_ptr(), l2.data_ptr(),
                                              2, 8, 16, 2, cas.CAS_F32, cas.CAS_F32, cas._stream_ptr(buf.device))
    assert st == -7


def test_workload_attention_fused_full_size(orc):
    wl = synth.WORKLOADS["trimul_f32_B8_T1024_NH12_HS64"]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    worst = check_attention_fused(orc, qkv, "f32", B, T, NH, HS, wl.name,
                                  b_t=[(0, 0, 64), (3, 500, 540), (7, 960, 1024)])
    print(f"{wl.name} fused attention: sampled max err/tol {worst:.3g}")


def test_workload_attention_fused_bf16_full_size(orc):
    wl = synth.WORKLOADS["trimul_bf16_B4_T4096_NH25_HS64"]
    B, T, NH, HS = wl.dims
    (qkv,) = wl.inputs()
    worst = check_attention_fused(orc, qkv, wl.dtype, B, T, NH, HS, wl.name,
                                  b_t=[(0, 0, 32), (2, 2040, 2060), (3, 4070, 4096)])
    print(f"{wl.name} fused attention: sampled max err/tol {worst:.3g}")


# --------------------------------------------------- general shapes
#
# Heads whose rows do not split into 16-byte pieces (HS = 3 and 5 in fp32,
# 12 in binary16, a base one element off alignment) or exceed 512 bytes
# (HS = 160 in fp32; 161 and 333 in fp32 and 336 in bfloat16, staged in two
# or three chunks of at most 640 bytes) run on the general-shape kernels. Heads of 257 .. 512
# bytes in 16-byte pieces (fp32 HS = 80, bf16 HS = 136) take the fast
# kernels' wide variants (32 pieces per row) and, for the softmax rows, the
# per-wave tile kernel with the softmax epilogue: the wide-head tests below.

GENERAL = [("f32", 3), ("f32", 5), ("f32", 160), ("f32", 161), ("f32", 333), ("f16", 12), ("bf16", 3),
           ("bf16", 336)]
GENERAL_ATT = GENERAL
GENERAL_T = [1, 33, 64, 100, 300]


@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("T", GENERAL_T)
@pytest.mark.parametrize("dtype,HS", GENERAL, ids=lambda v: str(v))
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_general_shapes(orc, launch, dtype, HS, T, mode):
    B, NH = 2, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 19 + HS)
    check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="general", launch=launch)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype,HS", [("f32", 160), ("f32", 3)], ids=lambda v: str(v))
def test_softmax_general_out16(orc, dtype, HS, out_dtype):
    B, T, NH = 2, 130, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 7)
    for mode in ("prob", "log"):
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, out_dtype, label="general out16", launch="fused")


KERNELS = ["fast", "general"]


def use_kernels(monkeypatch, kernel):
    if kernel == "general":
        monkeypatch.setenv("CAS_SOFTMAX_KERNEL", "general")
    else:
        monkeypatch.delenv("CAS_SOFTMAX_KERNEL", raising=False)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_misaligned_base(orc, monkeypatch, launch, dtype, kernel):
    """HS = 64 with qkv one element past a 16-byte boundary: the fast
    kernels (16-byte pieces at the base's offset) and the general ones."""
    use_kernels(monkeypatch, kernel)
    B, T, NH, HS = 2, 150, 2, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=23)
    for mode in ("prob", "log"):
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, label=f"misaligned base {kernel}", launch=launch,
                   qkv_offset=1)


@pytest.mark.parametrize("T", GENERAL_T)
@pytest.mark.parametrize("dtype,HS", GENERAL_ATT, ids=lambda v: str(v))
def test_attention_general_shapes(orc, dtype, HS, T):
    """Both attention paths on general shapes: the two-pass launches, and the
    one-launch entry point, which there computes the statistics first (two
    sweeps over the keys) and then y as the two-pass path does -- so it is
    held to the two-pass bound, and its row maxima to the statistics
    launch's, bit for bit."""
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 29 + HS)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "general two-pass")
    y, mx, ls = run_attention_fused(qkv, dtype, B, T, NH, HS, "general one launch")
    mx2, ls2 = cas.causal_row_stats(to_device(qkv, dtype).view(B, T, 3 * NH * HS), NH)
    assert np.array_equal(mx.view(np.uint32), mx2.cpu().numpy().view(np.uint32)), "row_max differs"
    assert np.array_equal(ls.view(np.uint32), ls2.cpu().numpy().view(np.uint32)), "row_logsum differs"
    check_attention(orc, qkv, dtype, B, T, NH, HS, "general one launch", y=y)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129, 300])
@pytest.mark.parametrize("HS", [68, 80, 128])
def test_attention_wide_heads_f32(orc, HS, T):
    """fp32 heads of 257 .. 512 bytes (32 pieces per row): the two-pass
    attention (statistics launch, then y) and the single pass, on the fast
    kernels; row maxima bit for bit against the statistics launch."""
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, "f32", seed=T * 37 + HS)
    check_attention(orc, qkv, "f32", B, T, NH, HS, "wide heads two-pass")
    check_attention_fused(orc, qkv, "f32", B, T, NH, HS, "wide heads")


@pytest.mark.parametrize("T", [1, 64, 65, 300])
@pytest.mark.parametrize("HS", [136, 192, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attention_wide_heads_16bit(orc, dtype, HS, T):
    """16-bit heads of 257 .. 512 bytes (32 pieces per row, kernels built with
    their output accumulators in the accumulation registers): both attention
    paths against the oracle, row maxima bit for bit against the statistics
    launch."""
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 43 + HS)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "wide heads two-pass")
    check_attention_fused(orc, qkv, dtype, B, T, NH, HS, "wide heads")


WIDE_SM = [("f32", 68), ("f32", 80), ("f32", 128), ("bf16", 136), ("bf16", 256), ("f16", 192)]


@pytest.mark.parametrize("mode", ["prob", "log"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 129, 300])
@pytest.mark.parametrize("dtype,HS", WIDE_SM, ids=lambda v: str(v))
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_wide_heads(orc, launch, dtype, HS, T, mode):
    """Heads of 257 .. 512 bytes (three or four 128-byte register passes):
    the wide statistics launch and the tile kernel's softmax rows, as two
    launches and through the fused entry point (the same two launches)."""
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=T * 53 + HS)
    check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="wide heads", launch=launch)


@pytest.mark.parametrize("dtype,HS", [("f32", 100), ("f32", 80), ("bf16", 256), ("bf16", 136)], ids=lambda v: str(v))
def test_softmax_wide_heads_kernels_agree(orc, monkeypatch, dtype, HS):
    """The wide-head softmax rows from the super-tile kernel (two head
    halves) equal those of the per-wave tile kernel bit for bit, both
    modes, fp32 and bf16 output."""
    B, T, NH = 2, 200, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 29)
    for mode in ("prob", "log"):
        for out_dtype in ("f32", "bf16"):
            got = {}
            for kernel in ("super", "tile"):
                if kernel == "tile":
                    monkeypatch.setenv("CAS_TRIMUL_KERNEL", "tile")
                else:
                    monkeypatch.delenv("CAS_TRIMUL_KERNEL", raising=False)
                got[kernel] = run_softmax(qkv, dtype, B, T, NH, HS, mode, out_dtype, f"kernels agree {kernel}")
            for a, b in zip(got["super"], got["tile"]):
                assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), \
                    f"{mode} {out_dtype}: kernels differ"
    monkeypatch.delenv("CAS_TRIMUL_KERNEL", raising=False)
    check_case(orc, qkv, dtype, B, T, NH, HS, "prob", label="wide heads super")


@pytest.mark.parametrize("dtype,HS", [("f32", 128), ("f32", 80), ("bf16", 256)], ids=lambda v: str(v))
def test_softmax_wide_heads_many_items(orc, monkeypatch, dtype, HS):
    """Wide-head softmax rows over many super-tiles per workgroup (B2 T1024
    NH8): bit for bit against the tile kernel, both modes, fp32 and bf16
    output, and sampled rows of the plane against the oracle."""
    B, T, NH = 2, 1024, 8
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 83)
    for mode in ("prob", "log"):
        for out_dtype in ("f32", "bf16"):
            got = {}
            for kernel in ("super", "tile"):
                if kernel == "tile":
                    monkeypatch.setenv("CAS_TRIMUL_KERNEL", "tile")
                else:
                    monkeypatch.delenv("CAS_TRIMUL_KERNEL", raising=False)
                got[kernel] = run_softmax(qkv, dtype, B, T, NH, HS, mode, out_dtype, f"many items {kernel}")
            for a, b in zip(got["super"], got["tile"]):
                assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), \
                    f"{mode} {out_dtype}: kernels differ"
    monkeypatch.delenv("CAS_TRIMUL_KERNEL", raising=False)
    out, mx, ls = run_softmax(qkv, dtype, B, T, NH, HS, "prob", "f32", "many items oracle rows")
    for b, h, t0 in [(0, 0, 0), (1, 5, 500), (1, 7, 992)]:
        ref, mref, lref, bound = orc.causal_softmax_rows(qkv, B, T, NH * HS, NH, b, h, t0, t0 + 32, dtype, "prob")
        r0 = (b * NH + h) * T + t0
        t_idx = np.arange(t0, t0 + 32)
        what = f"many items {dtype} HS={HS} b={b} h={h} t0={t0}"
        assert_softmax_stats(mx[r0:r0 + 32], ls[r0:r0 + 32], mref, lref, bound, t_idx, dtype, what)
        assert_softmax(out[r0:r0 + 32], ref, lref, bound, t_idx, dtype, "prob", "f32", what)


@pytest.mark.parametrize("T", [130, 200])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype,HS", [("f32", 80), ("bf16", 136)], ids=lambda v: str(v))
def test_softmax_wide_heads_out16(orc, dtype, HS, out_dtype, T):
    """16-bit output rows: per-element stores (T = 130) and 16-byte stores
    (T = 200, rows in 16-byte pieces)."""
    B, NH = 2, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 11)
    for mode in ("prob", "log"):
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, out_dtype, label="wide heads out16", launch="two")


@pytest.mark.parametrize("dtype,HS", [("f32", 96), ("f32", 100), ("bf16", 136)], ids=lambda v: str(v))
@pytest.mark.parametrize("offset", [0, 1])
def test_softmax_wide_heads_unaligned_output(orc, offset, dtype, HS):
    """Output rows not in 16-byte pieces (T = 97, and a base one element
    off): the masked per-element stores of the tile kernel (fp32 HS 96) and
    of the super-tile kernel in two head halves (fp32 HS 100, bf16 HS 136)."""
    B, T, NH = 1, 97, 3
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=59 + HS)
    for mode in ("prob", "log"):
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="wide heads unaligned", offset=offset)
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, "bf16", label="wide heads unaligned", offset=offset)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("launch", LAUNCHES)
def test_softmax_wide_heads_saturated_ramp(orc, launch, dtype):
    """Exact-score saturated ramp rows on 512-byte heads (HS = 256, scale
    1/16 exact): only the exp / log / sum roundings are allowed."""
    B, T, NH, HS = 1, 257, 4, 256
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [16.0 * a for a in SAT_SLOPES], dtype)
    for mode in ("prob", "log"):
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="wide ramp", exact_scores=True, launch=launch)


@pytest.mark.parametrize("dtype,HS", [("f32", 128), ("bf16", 136), ("f16", 256)], ids=lambda v: str(v))
def test_softmax_wide_heads_stats_match_the_score_kernel(orc, dtype, HS):
    """Wide heads: the statistics launch and the tile kernel form every
    score alike, bit for bit (row maxima equal the largest scores of
    cas_trimul_causal's rows, and the largest log-probability of a row is
    exactly -row_logsum)."""
    B, T, NH = 2, 200, 2
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=HS + 3)
    d = to_device(qkv, dtype).view(B, T, -1)
    case(f"wide stats vs scores {dtype} HS={HS}")
    sc = cas.trimul_causal(d, NH)
    low = torch.tril(torch.ones(T, T, dtype=torch.bool, device="cuda"))
    smax = torch.where(low, sc, torch.full_like(sc, -float("inf"))).amax(dim=-1)
    lp, mx, ls = cas.causal_softmax(d, NH, "log", fused=False)
    torch.cuda.synchronize()
    assert torch.equal(smax.view(torch.int32), mx.view(torch.int32)), "row_max"
    assert torch.equal(lp.amax(dim=-1).view(torch.int32), (-ls).view(torch.int32)), "max lp"


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_attention_misaligned_base(orc, monkeypatch, dtype, kernel):
    use_kernels(monkeypatch, kernel)
    B, T, NH, HS = 2, 97, 2, 64
    qkv = synth.trimul_inputs(B, T, NH, HS, dtype, seed=31)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "misaligned base", qkv_offset=1)
    y, _, _ = run_attention_fused(qkv, dtype, B, T, NH, HS, "misaligned base one launch", qkv_offset=1)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "misaligned base one launch", y=y)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_general_saturated_ramp(orc, monkeypatch, dtype, kernel):
    """Exact-score saturated rows (slopes 64, -16, 0.25, 200) with a base one
    element off alignment, on the general kernels and on the fast ones (HS =
    64, where the scale 1/8 keeps every score exact): statistics,
    probabilities and the attention output pinned to exp / sum roundings
    only."""
    use_kernels(monkeypatch, kernel)
    B, T, NH, HS = 1, 257, 4, 64
    qkv = synth.ramp_qk_inputs(B, T, NH, HS, [8.0 * a for a in SAT_SLOPES], dtype, v_seed=47)
    for mode in ("prob", "log"):
        check_case(orc, qkv, dtype, B, T, NH, HS, mode, label="general ramp", exact_scores=True, launch="two",
                   qkv_offset=1)
    check_attention(orc, qkv, dtype, B, T, NH, HS, "general ramp", exact_scores=True, qkv_offset=1)
