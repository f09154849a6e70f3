"""The C ABI on a machine without a GPU: the library loads, exports every
symbol include/cas.h declares, and rejects bad arguments before any HIP call."""
import os
import re

import pytest

import causal_attention_score_amd as cas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cas.h")

F32, BF16, F16 = cas.CAS_F32, cas.CAS_BF16, cas.CAS_F16
OK, ENULL, ESHAPE, EDTYPE, EALIAS, EDEV = 0, -1, -2, -3, -4, -5
EUNSUP, EMODE = -7, -8

# Fake, distinct, aligned addresses: validation never dereferences them.
PX, PW, PY, PZ = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cas.LIB_PATH):
        pytest.skip("libcas.so not built")
    return cas.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cas_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(cas.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in list(cas.STATUS) + [7, -99]:
        s = cas.status_string(code)
        assert isinstance(s, str) and s
    assert L.cas_version() >= 100


def g(L, X=PX, W=PW, Y=PY, M=4, N=5, K=6, ldx=None, ldw=None, ldy=None, ind=F32, outd=F32):
    return L.cas_gemm_nt(X, W, Y, M, N, K, K if ldx is None else ldx, K if ldw is None else ldw,
                         N if ldy is None else ldy, ind, outd, None)


def bm(L, X=PX, W=PW, Y=PY, batch=3, M=4, N=5, K=6, ldx=None, ldw=None, ldy=None, bsx=None, bsw=None, bsy=None,
       ind=F32, outd=F32):
    ldx = K if ldx is None else ldx
    ldw = K if ldw is None else ldw
    ldy = N if ldy is None else ldy
    return L.cas_batch_matmul_nt(X, W, Y, batch, M, N, K, ldx, ldw, ldy,
                                 M * ldx if bsx is None else bsx, N * ldw if bsw is None else bsw,
                                 M * ldy if bsy is None else bsy, ind, outd, None)


def t(L, qkv=PX, out=PY, B=2, T=5, C=12, NH=3, ind=F32, outd=F32):
    return L.cas_trimul_causal(qkv, out, B, T, C, NH, ind, outd, None)


def rs(L, qkv=PX, mx=PY, ls=PW, B=2, T=5, C=12, NH=3, ind=F32):
    return L.cas_causal_row_stats(qkv, mx, ls, B, T, C, NH, ind, None)


def sm(L, qkv=PX, mx=PY, ls=PW, out=PZ, B=2, T=5, C=12, NH=3, mode=1, ind=F32, outd=F32):
    return L.cas_causal_softmax(qkv, mx, ls, out, B, T, C, NH, mode, ind, outd, None)


def test_gemm_rejections(L):
    assert g(L, ind=7) == EDTYPE
    assert g(L, outd=BF16) == EDTYPE
    assert g(L, M=-1) == ESHAPE
    assert g(L, K=-2) == ESHAPE
    assert g(L, ldx=5) == ESHAPE            # ldx < K
    assert g(L, ldw=3) == ESHAPE            # ldw < K
    assert g(L, ldy=4) == ESHAPE            # ldy < N
    assert g(L, Y=None) == ENULL
    assert g(L, X=None) == ENULL
    assert g(L, W=None) == ENULL
    assert g(L, Y=PX + 8) == EALIAS         # output starts inside X
    assert g(L, X=PY + 4 * 5 * 4 - 4) == EALIAS  # X starts at Y's last element
    assert g(L, M=2**40, ldx=2**40, K=6) == ESHAPE  # byte extent above 2^62
    assert g(L, M=2**62, N=4, K=4) == ESHAPE  # byte extent overflows


def test_gemm_empty_is_ok_without_a_device(L):
    assert g(L, M=0) == OK
    assert g(L, N=0, ldy=0) == OK
    assert g(L, X=None, W=None, Y=None, M=0) == OK


def test_gemm_k0_needs_no_inputs(L):
    # K == 0 writes zeros: X and W may be NULL; with no GPU the call stops at
    # the device check.
    assert g(L, X=None, W=None, K=0) == EDEV


def test_batch_matmul_rejections(L):
    assert bm(L, ind=9) == EDTYPE
    assert bm(L, outd=F16) == EDTYPE
    assert bm(L, batch=-1) == ESHAPE
    assert bm(L, bsx=-1) == ESHAPE
    assert bm(L, ldy=4) == ESHAPE
    assert bm(L, bsy=4 * 5 - 1) == ESHAPE   # output blocks would overlap
    assert bm(L, Y=None) == ENULL
    assert bm(L, W=None) == ENULL
    assert bm(L, Y=PX + 2 * 4 * 6 * 4) == EALIAS   # output starts inside the third X block
    assert bm(L, X=PY + 2 * 4 * 5 * 4, bsx=0) == EALIAS  # X inside the last output block
    assert bm(L, batch=2**40, bsy=2**30) == ESHAPE      # byte extent above 2^62


def test_batch_matmul_empty_and_broadcast_reach_the_device_check(L):
    import torch
    assert bm(L, batch=0) == OK
    assert bm(L, M=0) == OK
    assert bm(L, X=None, W=None, Y=None, batch=0) == OK
    if not torch.cuda.is_available():
        assert bm(L, bsw=0) == EDEV     # one W block for every batch: valid
        assert bm(L, batch=1, bsy=0) == EDEV


def test_trimul_rejections(L):
    assert t(L, ind=3) == EDTYPE
    assert t(L, outd=7) == EDTYPE
    assert t(L, B=-1) == ESHAPE
    assert t(L, C=10, NH=3) == ESHAPE       # C % NH != 0
    assert t(L, C=0) == ESHAPE
    assert t(L, qkv=None) == ENULL
    assert t(L, out=None) == ENULL
    assert t(L, out=PX + 64) == EALIAS
    assert t(L, B=2**40, T=2**20) == ESHAPE
    assert t(L, B=1, T=2**24, C=12, NH=3) == ESHAPE   # T at the 32-bit offset limit
    assert t(L, B=1, T=4, C=2**22, NH=2) == ESHAPE    # QKV row of 3 * 2^24 fp32 bytes


def test_trimul_16bit_outputs(L):
    import torch
    # (B, NH, T, T) = (2, 3, 5, 5) outputs of 2 bytes span 300 bytes: qkv
    # starting 298 bytes past the output overlaps it, 300 bytes past does not
    # (with fp32 outputs, 600 bytes, it would).
    assert t(L, qkv=PY + 298, outd=BF16) == EALIAS
    assert t(L, qkv=PY + 300, outd=F32) == EALIAS
    if not torch.cuda.is_available():
        assert t(L, outd=BF16) == EDEV
        assert t(L, outd=F16, ind=BF16) == EDEV
        assert t(L, qkv=PY + 300, outd=F16) == EDEV


def test_trimul_empty_is_ok(L):
    assert t(L, B=0) == OK
    assert t(L, T=0) == OK
    assert t(L, NH=0, C=0) == OK


def fu(L, qkv=PX, mx=PY, ls=PW, out=PZ, B=2, T=5, C=12, NH=3, mode=1, ind=F32, outd=F32):
    return L.cas_causal_softmax_fused(qkv, out, mx, ls, B, T, C, NH, mode, ind, outd, None)


def at(L, qkv=PX, mx=PY, ls=PW, y=PZ, B=2, T=5, C=12, NH=3, ind=F32, outd=F32):
    return L.cas_causal_attention(qkv, mx, ls, y, B, T, C, NH, ind, outd, None)


def test_attention_rejections(L):
    import torch
    assert at(L, ind=5) == EDTYPE
    assert at(L, outd=BF16) == EDTYPE
    assert at(L, B=-1) == ESHAPE
    assert at(L, C=10, NH=3) == ESHAPE
    assert at(L, y=None) == ENULL and at(L, qkv=None) == ENULL and at(L, mx=None) == ENULL
    assert at(L, qkv=PX + 2) == EUNSUP                      # fp32 elements off their 4-byte alignment
    assert at(L, y=PX + 16) == EALIAS                       # y inside qkv
    assert at(L, y=PY + 64) == EALIAS                       # y over the statistics
    assert at(L, B=0) == OK and at(L, T=0) == OK
    if not torch.cuda.is_available():
        assert at(L) == EDEV
        assert at(L, mx=PX + 16, ls=PX + 32) == EDEV        # the statistics are only read
        assert at(L, ind=BF16, C=24) == EDEV                # 16-byte heads of a 16-bit type
        # general shapes: accepted, served by the general-shape kernels
        assert at(L, ind=F16, C=12) == EDEV                 # 8-byte heads of a 16-bit type
        assert at(L, C=15, NH=3) == EDEV                    # 20-byte heads
        assert at(L, C=3 * 160, NH=3) == EDEV               # HS = 160 fp32: 640-byte heads
        assert at(L, C=3 * 161, NH=3) == EDEV               # HS = 161 fp32: 644-byte heads, staged in chunks
        assert at(L, ind=F16, C=3 * 336, NH=3) == EDEV      # HS = 336 binary16: 672-byte heads
        assert at(L, B=2**23, T=1, C=4, NH=1) == EDEV       # past the fast kernels' grid limits


def af(L, qkv=PX, y=PZ, mx=PY, ls=PW, B=2, T=5, C=12, NH=3, ind=F32, outd=F32):
    return L.cas_causal_attention_fused(qkv, y, mx, ls, B, T, C, NH, ind, outd, None)


def test_attention_fused_rejections(L):
    import torch
    assert af(L, ind=5) == EDTYPE
    assert af(L, outd=BF16) == EDTYPE
    assert af(L, B=-1) == ESHAPE
    assert af(L, C=10, NH=3) == ESHAPE
    assert af(L, y=None) == ENULL and af(L, qkv=None) == ENULL and af(L, mx=None) == ENULL
    assert af(L, ls=None) == ENULL
    assert af(L, qkv=PX + 2) == EUNSUP                      # fp32 elements off their alignment
    assert af(L, mx=PY + 2) == EUNSUP and af(L, y=PZ + 2) == EUNSUP
    # three outputs: none over qkv or over another; (B, T, C) fp32 y spans 480 bytes, statistics 120
    assert af(L, y=PX + 16) == EALIAS
    assert af(L, mx=PX + 16) == EALIAS
    assert af(L, y=PY - 256) == EALIAS                      # y over row_max
    assert af(L, ls=PY + 116) == EALIAS                     # row_logsum over row_max's last value
    assert af(L, B=0) == OK and af(L, T=0) == OK
    assert af(L, qkv=None, y=None, mx=None, ls=None, B=0) == OK
    if not torch.cuda.is_available():
        assert af(L) == EDEV
        assert af(L, y=PZ + 4) == EDEV                      # 4-byte aligned y: scalar stores
        assert af(L, ind=BF16, C=24) == EDEV
        assert af(L, ind=F16, C=12) == EDEV                 # general shapes
        assert af(L, C=15, NH=3) == EDEV
        assert af(L, C=3 * 161, NH=3) == EDEV               # heads over 640 bytes, staged in chunks
        assert af(L, B=2**23, T=1, C=4, NH=1) == EDEV


def test_softmax_rejections(L):
    for f in (rs, sm, fu):
        assert f(L, ind=5) == EDTYPE
        assert f(L, B=-1) == ESHAPE
        assert f(L, C=10, NH=3) == ESHAPE
        assert f(L, qkv=None) == ENULL
        assert f(L, mx=None) == ENULL
        assert f(L, ls=None) == ENULL
        assert f(L, B=2**40, T=2**20) == ESHAPE
        assert f(L, B=1, T=4, C=2**22, NH=2) == ESHAPE
        # outside both the fast and the general kernels' domains (valid arguments otherwise)
        assert f(L, qkv=PX + 2) == EUNSUP                  # fp32 elements off their 4-byte alignment
        assert f(L, mx=PY + 2) == EUNSUP                   # misaligned statistics
        assert f(L, B=0) == OK and f(L, T=0) == OK and f(L, NH=0, C=0) == OK
        assert f(L, qkv=None, mx=None, ls=None, B=0) == OK
    for f in (sm, fu):
        assert f(L, out=None) == ENULL
        assert f(L, mode=2) == EMODE and f(L, mode=-1) == EMODE
        assert f(L, outd=9) == EDTYPE
    # the fused call writes all three: no overlap among them or with qkv
    assert fu(L, mx=PX + 16) == EALIAS
    assert fu(L, ls=PY + 116) == EALIAS
    assert fu(L, out=PY) == EALIAS
    assert fu(L, mx=PZ + 64) == EALIAS
    # (B, NH, T) statistics of 4 bytes span 120 bytes.
    assert rs(L, mx=PX + 16) == EALIAS                      # statistics inside qkv
    assert rs(L, ls=PY + 116) == EALIAS                     # row_logsum over row_max's last value
    assert sm(L, out=PY + 64) == EALIAS                     # output over the statistics it reads
    assert sm(L, out=PX + 64) == EALIAS                     # output over qkv
    assert sm(L, qkv=PZ + 288, outd=BF16) == EALIAS      # 16-bit output spans 300 bytes


def test_softmax_valid_calls_reach_the_device_check(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert rs(L) == EDEV
    assert rs(L, ind=BF16, C=3 * 128, NH=3) == EDEV        # 256-byte heads: the largest accepted
    assert sm(L) == EDEV
    assert sm(L, mode=0, outd=BF16, ind=F16, C=24) == EDEV  # HS = 8: 16-byte heads
    assert sm(L, qkv=PZ + 304, outd=F16) == EDEV           # qkv (aligned) after the 300-byte output
    assert sm(L, mx=PX + 16) == EDEV                       # statistics may overlap qkv when read
    assert fu(L) == EDEV
    assert fu(L, mode=0, outd=F16, ind=BF16, C=24) == EDEV
    # general shapes reach the device check too
    for f in (rs, sm, fu):
        assert f(L, qkv=PX + 4) == EDEV                    # QKV rows not in 16-byte pieces
        assert f(L, C=15, NH=3) == EDEV                    # HS = 5 fp32: 20-byte heads
        assert f(L, C=3 * 80, NH=3, ind=F32) == EDEV       # HS = 80 fp32: 320-byte heads
        assert f(L, C=3 * 136, NH=3, ind=BF16) == EDEV     # HS = 136 bf16: 272-byte heads
        assert f(L, C=3 * 160, NH=3, ind=F32) == EDEV      # HS = 160 fp32: 640-byte heads, one chunk
        assert f(L, C=3 * 161, NH=3, ind=F32) == EDEV      # HS = 161 fp32: two chunks
        assert f(L, C=3 * 336, NH=3, ind=BF16) == EDEV     # HS = 336 bf16: 672-byte heads
        assert f(L, C=3 * 1024, NH=3, ind=F32) == EDEV     # HS = 1024 fp32: 4 KB heads
        assert f(L, B=1, T=2**22, C=12, NH=3) == EDEV      # past the fast kernels' T limit
        assert f(L, B=2**23, T=1, C=4, NH=1) == EDEV       # past the fast kernels' grid limits


def test_valid_calls_reach_the_device_check(L):
    # On a machine with no GPU a valid call fails at the device check only.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert g(L) == EDEV
    assert t(L) == EDEV


def test_binding_validates_shapes():
    import torch
    x = torch.zeros(3, 4)
    with pytest.raises(ValueError):
        cas.gemm_nt(x, torch.zeros(5, 3))
    with pytest.raises(TypeError):
        cas.gemm_nt(x, torch.zeros(5, 4, dtype=torch.float16))
    with pytest.raises(ValueError):
        cas.trimul_causal(torch.zeros(2, 3, 10), 2)
    with pytest.raises(ValueError):
        cas.causal_softmax(torch.zeros(2, 3, 12), 3, mode="softmax")
    with pytest.raises(ValueError):
        cas.causal_row_stats(torch.zeros(2, 3, 10), 2)


@pytest.mark.parametrize("bad", ["dtype", "shape", "strided"])
def test_binding_validates_attention_stats(bad):
    """causal_attention(stats=...) hands the two pointers to a kernel that reads
    B*NH*T floats from each: a wrong dtype, shape or layout is rejected before
    any call reaches the library."""
    import torch
    B, T, NH, HS = 2, 8, 2, 4
    qkv = torch.zeros(B, T, 3 * NH * HS)
    good = torch.zeros(B, NH, T)
    if bad == "dtype":
        wrong = torch.zeros(B, NH, T, dtype=torch.float16)
    elif bad == "shape":
        wrong = torch.zeros(B, NH, T - 1)
    else:
        wrong = torch.zeros(B, NH, 2 * T)[..., ::2]
    for stats in ((wrong, good), (good, wrong)):
        with pytest.raises(ValueError, match="row_max / row_logsum"):
            cas.causal_attention(qkv, NH, stats=stats)
