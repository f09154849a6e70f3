"""The entry points under HIP graph capture. The library allocates nothing,
never synchronises and records no memset, so a sequence of its calls can be
captured once on a stream and replayed. Each replay must reproduce the eager
results bit for bit (the kernels are deterministic); between replays the
outputs are overwritten by eager work of the program's own, with
synchronisations, so a replay that skipped a kernel or wrote stale data
would show."""
import pytest
import torch

import causal_attention_score_amd as cas
from causal_attention_score_amd import synth
from gpu_util import assert_close, case, to_device

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_hot_path_replays_in_a_graph(orc):
    # dense fp32 960x1024x770 and the fp32 scores (the benchmark step's two
    # kernels), the two-launch fp32 softmax, the fused bf16 softmax to bf16,
    # and both attention forms
    X, W = synth.gemm_inputs(960, 1024, 770, "f32", seed=61)
    x, w = to_device(X, "f32"), to_device(W, "f32")
    B, T, NH, HS = 2, 300, 3, 64
    q = to_device(synth.trimul_inputs(B, T, NH, HS, "f32", seed=62), "f32").view(B, T, 3 * NH * HS)
    B2, T2, NH2 = 1, 257, 2
    q16 = to_device(synth.trimul_inputs(B2, T2, NH2, HS, "bf16", seed=63), "bf16").view(B2, T2, 3 * NH2 * HS)
    dev = q.device

    y = torch.empty(960, 1024, device=dev)
    sc = torch.empty(B, NH, T, T, device=dev)
    mx, ls = torch.empty(B, NH, T, device=dev), torch.empty(B, NH, T, device=dev)
    lp = torch.empty(B, NH, T, T, device=dev)
    p16 = torch.empty(B2, NH2, T2, T2, device=dev, dtype=torch.bfloat16)
    mx16, ls16 = torch.empty(B2, NH2, T2, device=dev), torch.empty(B2, NH2, T2, device=dev)
    att = torch.empty(B, T, NH * HS, device=dev)
    att16 = torch.empty(B2, T2, NH2 * HS, device=dev)
    amx16, als16 = torch.empty(B2, NH2, T2, device=dev), torch.empty(B2, NH2, T2, device=dev)
    outs = [y, sc, mx, ls, lp, p16, mx16, ls16, att, att16, amx16, als16]

    def step():
        cas.gemm_nt(x, w, out=y)
        cas.trimul_causal(q, NH, out=sc)
        cas.causal_row_stats(q, NH, row_max=mx, row_logsum=ls)
        cas.causal_softmax(q, NH, "log", out=lp, stats=(mx, ls))
        st = cas.lib().cas_causal_softmax_fused(q16.data_ptr(), p16.data_ptr(), mx16.data_ptr(), ls16.data_ptr(),
                                                B2, T2, NH2 * HS, NH2, cas.SOFTMAX_MODE["prob"], cas.CAS_BF16,
                                                cas.CAS_BF16, cas._stream_ptr(dev))
        assert st == 0, cas.status_string(st)
        cas.causal_attention(q, NH, y=att, stats=(mx, ls))
        cas.causal_attention_fused(q16, NH2, y=att16, row_max=amx16, row_logsum=als16)

    case("graph: eager reference")
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    # the eager dense product is also right, not only repeatable
    want, bound = orc.gemm_nt(X, W, "f32")
    assert_close(y.cpu().numpy(), want, bound, "f32", "eager dense product")

    case("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(3):
        # eager work between replays: every output overwritten, a torch
        # product on the same stream, a synchronisation
        for o in outs:
            _bits(o).fill_(-1 - i)
        _ = torch.mm(torch.randn(256, 256, device=dev), torch.randn(256, 256, device=dev))
        torch.cuda.synchronize()
        case(f"graph: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(o), _bits(r)), f"replay {i}: output {k} differs from the eager run"
