"""Throughput of the tiled-matmul hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * gemm_nt       fp32 X [960, 770] . W [1024, 770]^T (the DietCode dense layer
                  with H = 1024; N(0,1)/sqrt(770) inputs), and
  * trimul_causal fp32 causal scores from packed QKV (8, 1024, 3, 12, 64)
                  (the llm.c trimat_forward.cu benchmark shape; N(0,1)).

value = useful TFLOP/s of the step (2MNK for the dense product, the lower
triangle including the diagonal, 2*HS*B*NH*T(T+1)/2, for the scores), with
inputs resident in HBM. The JSON line also carries the roofline of the
dominant kernel (timed with HIP events on its own stream), the oracle's
throughput on the host cores, the bf16 workloads (4096^3 dense, causal
scores (4, 4096, 3, 25, 64)) timed the same way, and the local-padding A/B:
the fp32 dense layer at H = 1024 and at DietCode's H = 2304, with the bounds
checks removed from the MFMA loop (the product path) and kept there
(CAS_VARIANT=predicated).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-bf16] [--no-ab]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6}   # dense MFMA
METRIC = "useful TFLOP/s (gemm_nt, trimul_causal) + % of MI355X MFMA/HBM roofline"
# Warm-up of the headline step lasts at least this long: launches timed within
# the first few hundred milliseconds after the GPU leaves idle run slower while
# its clocks ramp up.
SETTLE_S = 0.5
SUB_SETTLE_S = 0.25   # the same for each further workload (inputs are made on the host in between)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def device_tensor(a, dtype):
    import numpy as np
    import torch
    if dtype == "f32":
        return torch.from_numpy(a).cuda()
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a.view(np.float16)).cuda()


# Sources each profiled kernel is built from (its translation unit, what it
# includes, and the host dispatch in front of it), keyed by the workload it is
# profiled on.
KERNEL_SOURCES = {
    "trimul_f32_B8_T1024_NH12_HS64": ["cas_api.hip", "launch.hpp", "tile_engine.hpp", "trimul.hip",
                                      "trimul_f32.hip", "trimul_kernel.hpp"],
    "dense_f32_960x1024x770": ["cas_api.hip", "launch.hpp", "tile_engine.hpp", "gemm_nt.hip", "gemm_nt_direct.hip"],
    "dense_bf16_4096": ["cas_api.hip", "launch.hpp", "tile_engine.hpp", "gemm_nt.hip", "gemm_nt_wide.hip"],
    "trimul_bf16_B4_T4096_NH25_HS64": ["cas_api.hip", "launch.hpp", "tile_engine.hpp", "trimul.hip",
                                       "trimul_bf16.hip", "trimul_kernel.hpp"],
}
# Workloads whose kernels the counter runs profile (bench.py --traffic-probe).
PROBED = tuple(KERNEL_SOURCES)


def kernel_sources_digest(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the sources `kernel` is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_attention_score_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def read_counters(kernel: str):
    """Counter figures of `kernel` from its committed rocprofv3 summary
    (profiles/counters_<workload>.md), if they were taken on the kernel's
    current sources; else None. Keys: hbm_bytes_per_launch (FETCH_SIZE and
    WRITE_SIZE, each scaled by what it reads for a plain copy of known size),
    and where measured mfma_busy_frac, wait_frac, lds_bank_conflict_frac,
    clock_ghz."""
    digest = kernel_sources_digest(kernel)
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("sources_digest") != digest:
        return None
    out = {}
    for k in ("hbm_bytes_per_launch", "mfma_busy_frac", "wait_frac", "lds_bank_conflict_frac", "clock_ghz"):
        try:
            out[k] = float(vals[k])
        except (KeyError, ValueError):
            pass
    return out or None


class Part:
    """One entry point on one workload, with device buffers ready."""

    def __init__(self, wl, out_dtype: str = "f32"):
        import torch

        import causal_attention_score_amd as cas
        self.wl = wl
        self.cas = cas
        self.out_dtype = out_dtype
        if wl.kind in ("gemm_nt", "batch_matmul_nt"):
            X, W = wl.inputs()
            self.x, self.w = device_tensor(X, wl.dtype), device_tensor(W, wl.dtype)
            shape = wl.dims[:2] if wl.kind == "gemm_nt" else (wl.dims[0], wl.dims[1], wl.dims[2])
            self.out = torch.empty(shape, dtype=torch.float32, device="cuda")
        else:
            (qkv,) = wl.inputs()
            B, T, NH, _ = wl.dims
            self.qkv = device_tensor(qkv, wl.dtype)
            self.NH = NH
            tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
            self.out = torch.empty((B, NH, T, T), dtype=tdt, device="cuda")

    def __call__(self):
        if self.wl.kind == "gemm_nt":
            self.cas.gemm_nt(self.x, self.w, out=self.out)
        elif self.wl.kind == "batch_matmul_nt":
            self.cas.batch_matmul_nt(self.x, self.w, out=self.out)
        else:
            self.cas.trimul_causal(self.qkv, self.NH, out=self.out)


def time_parts(parts, steps: int, warmup: int, settle_s: float = 0.0, per_launch: bool = True):
    """Warm up, then time `steps` steps (twice with several parts). The
    warm-up is `warmup` steps,
    continued (untimed) until `settle_s` seconds have passed, so the timed
    steps do not run while the GPU's clocks are still ramping up from idle.
    With several parts, the first timed pass brackets the steps with HIP
    events at its two ends only: the step time. The second pass runs the same
    steps with an event after every part, on the stream the parts are launched
    on: the per-part times (an event between two launches adds a dispatch gap,
    about 9 us per step for the two-kernel step, so these events stay out of
    the step time). A single part is timed in one pass with an event after
    every launch, or with per_launch=False like a step (events at the two
    ends only; the per-part figures are then the step's). Returns (ms per
    step, [mean ms per part], wall ms per step, [median ms per part], warm-up
    steps run)."""
    import torch
    stream = torch.cuda.current_stream()
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_warm < settle_s:
        for p in parts:
            p()
        done += 1
        if done >= warmup and done % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(steps)]
    single = len(parts) == 1 and per_launch
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(steps):
        if single:
            ev[s][0].record(stream)
        for p in parts:
            p()
        if single:
            ev[s][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    total = start.elapsed_time(stop)
    if len(parts) == 1 and not per_launch:
        return total / steps, [total / steps], wall / steps, [total / steps], done
    if not single:
        for s in range(steps):
            ev[s][0].record(stream)
            for i, p in enumerate(parts):
                p()
                ev[s][i + 1].record(stream)
        torch.cuda.synchronize()
    each = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)] for i in range(len(parts))]
    per = [sum(e) / steps for e in each]
    med = [statistics.median(e) for e in each]
    return total / steps, per, wall / steps, med, done


def roofline_of(wl, ms: float, counters=None, out_bytes: int = 4):
    """Roofline entry of one kernel from its average launch time. `counters`
    are the rocprofv3 figures committed under profiles/ for this kernel's
    current sources (read_counters), or None. `traffic` is their HBM bytes per
    launch over the same launch time, in GB/s (the unit of `achieved` when the
    bound is HBM); `traffic_over_algorithmic` compares the bytes themselves.
    `counters` also carries MFMA-busy and wait fractions where measured."""
    t = ms * 1e-3
    tb = counters.get("hbm_bytes_per_launch") if counters else None
    traffic = round(tb / t / 1e9, 1) if tb else None
    extra = {"traffic": traffic, "traffic_bytes_per_launch": tb,
             "counters": {k: v for k, v in counters.items() if k != "hbm_bytes_per_launch"} if counters else None}
    if wl.kind == "trimul_causal":
        achieved = wl.algorithmic_bytes(out_bytes) / t / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), **extra,
                "traffic_over_algorithmic": round(tb / wl.algorithmic_bytes(out_bytes), 4) if tb else None,
                "kernel": f"trimul_causal {wl.name}", "avg_launch_us": round(ms * 1e3, 2),
                "algorithmic_bytes": wl.algorithmic_bytes(out_bytes)}
    achieved = wl.useful_flops() / t / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), **extra,
            "traffic_over_algorithmic": round(tb / wl.algorithmic_bytes(), 4) if tb else None,
            "kernel": f"gemm_nt {wl.name}", "avg_launch_us": round(ms * 1e3, 2),
            "useful_flops": wl.useful_flops(), "algorithmic_bytes": wl.algorithmic_bytes()}


class SoftmaxParts:
    """The two launches of the causal softmax (row statistics, softmax rows)
    on one score workload, with device buffers ready."""

    def __init__(self, wl, mode: str, out_dtype: str):
        import torch

        import causal_attention_score_amd as cas
        (qkv,) = wl.inputs()
        B, T, NH, _ = wl.dims
        self.cas, self.NH, self.mode = cas, NH, mode
        self.dims = (B, T, NH * wl.dims[3], NH)
        self.y = None
        self.qkv = device_tensor(qkv, wl.dtype)
        self.mx = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
        self.ls = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
        self.out = torch.empty((B, NH, T, T), dtype=tdt, device="cuda")

    def stats(self):
        self.cas.causal_row_stats(self.qkv, self.NH, row_max=self.mx, row_logsum=self.ls)

    def rows(self):
        self.cas.causal_softmax(self.qkv, self.NH, self.mode, out=self.out, stats=(self.mx, self.ls))

    def attention(self):
        if self.y is None:
            import torch
            B, T, C, _ = self.dims
            self.y = torch.empty((B, T, C), dtype=torch.float32, device="cuda")
        self.cas.causal_attention(self.qkv, self.NH, y=self.y, stats=(self.mx, self.ls))

    def attention_fused(self):
        if self.y is None:
            import torch
            B, T, C, _ = self.dims
            self.y = torch.empty((B, T, C), dtype=torch.float32, device="cuda")
        self.cas.causal_attention_fused(self.qkv, self.NH, y=self.y, row_max=self.mx, row_logsum=self.ls)

    def fused(self):
        L = self.cas.lib()
        st = L.cas_causal_softmax_fused(self.qkv.data_ptr(), self.out.data_ptr(), self.mx.data_ptr(),
                                        self.ls.data_ptr(), *self.dims, self.cas.SOFTMAX_MODE[self.mode],
                                        self.cas._dtype_code(self.qkv), self.cas._dtype_code(self.out),
                                        self.cas._stream_ptr(self.qkv.device))
        self.cas._check("cas_causal_softmax_fused", st)


def softmax_timings(steps: int):
    """The causal softmax fused on the scores (both launches recompute Q K^T
    from packed QKV; the (T, T) scores never reach HBM) on the two score
    shapes. Row statistics: bounded by the MFMA work (fp32) or by the one
    exp2 per score (16-bit inputs); softmax rows: HBM-bound like the scores
    (Q and K read, statistics read, every output written once)."""
    import torch

    from causal_attention_score_amd import synth
    out = {}
    for name, mode, od in (("trimul_f32_B8_T1024_NH12_HS64", "prob", "f32"),
                           ("trimul_f32_B8_T1024_NH12_HS64", "log", "f32"),
                           ("trimul_bf16_B4_T4096_NH25_HS64", "prob", "bf16"),
                           ("trimul_bf16_B4_T4096_NH25_HS64", "prob", "f32")):
        wl = synth.WORKLOADS[name]
        B, T, NH, HS = wl.dims
        key = f"{name}_{mode}_out_{od}"
        log(f"softmax timing {key}")
        sp = SoftmaxParts(wl, mode, od)
        n = max(5, steps // (10 if T > 2048 else 2))
        ms_step, (ms_st, ms_rows), _, _, _ = time_parts([sp.stats, sp.rows], n, 2, SUB_SETTLE_S)
        _, (ms_fused,), _, _, _ = time_parts([sp.fused], n, 2, SUB_SETTLE_S)
        # the fused launch timed like the two-launch step (events at the ends
        # only), for a like-for-like comparison of the two paths
        ms_fused_step, _, _, _, _ = time_parts([sp.fused], n, 2, SUB_SETTLE_S, per_launch=False)
        ob = 4 if od == "f32" else 2
        rows_bytes = wl.algorithmic_bytes(ob) + 8 * B * NH * T
        st_bytes = wl.algorithmic_bytes(0) + 8 * B * NH * T
        scores = B * NH * T * (T + 1) // 2
        out[key] = {
            "step_us": round(ms_step * 1e3, 2),
            "fused": {"avg_launch_us": round(ms_fused * 1e3, 2), "step_us": round(ms_fused_step * 1e3, 2),
                      "roofline": {"bound": "hbm", "achieved": round(rows_bytes / (ms_fused * 1e-3) / 1e9, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(rows_bytes / (ms_fused * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "algorithmic_bytes": rows_bytes}},
            "row_stats": {"avg_launch_us": round(ms_st * 1e3, 2),
                          "useful_tflops": round(wl.useful_flops() / (ms_st * 1e-3) / 1e12, 2),
                          "mfma_frac": round(wl.useful_flops() / (ms_st * 1e-3) / 1e12 / PEAK_TFLOPS[wl.dtype], 4),
                          "exp_per_ns": round(scores / (ms_st * 1e6), 1),
                          "hbm_gbs": round(st_bytes / (ms_st * 1e-3) / 1e9, 1)},
            "softmax_rows": {"avg_launch_us": round(ms_rows * 1e3, 2),
                             "roofline": {"bound": "hbm", "achieved": round(rows_bytes / (ms_rows * 1e-3) / 1e9, 1),
                                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                          "frac": round(rows_bytes / (ms_rows * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                          "algorithmic_bytes": rows_bytes}},
        }
        if mode == "prob" and od == "f32":
            # the attention output: softmax probabilities times V (statistics from the launch above)
            _, (ms_att,), _, _, _ = time_parts([sp.attention], n, 2, SUB_SETTLE_S)
            flops = 2 * wl.useful_flops()  # Q K^T and P V over the causal triangle
            out[key]["attention"] = {
                "avg_launch_us": round(ms_att * 1e3, 2),
                "with_row_stats_us": round((ms_att + ms_st) * 1e3, 2),
                "roofline": {"bound": "mfma", "achieved": round(flops / (ms_att * 1e-3) / 1e12, 2),
                             "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                             "frac": round(flops / (ms_att * 1e-3) / 1e12 / PEAK_TFLOPS[wl.dtype], 4),
                             "useful_flops": flops}}
            # the same output and the statistics in one pass (running maximum and sum)
            _, (ms_one,), _, _, _ = time_parts([sp.attention_fused], n, 2, SUB_SETTLE_S)
            out[key]["attention_single_pass"] = {
                "avg_launch_us": round(ms_one * 1e3, 2),
                "roofline": {"bound": "mfma", "achieved": round(flops / (ms_one * 1e-3) / 1e12, 2),
                             "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                             "frac": round(flops / (ms_one * 1e-3) / 1e12 / PEAK_TFLOPS[wl.dtype], 4),
                             "useful_flops": flops}}
        del sp
        torch.cuda.empty_cache()
    return out


def local_padding_ab(steps: int):
    """The dense fp32 layer with local padding (predicates only at fetch and
    writeback) against the same kernel with the bounds checks kept inside the
    MFMA loop (CAS_VARIANT=predicated), on the 1024-wide layer, on the
    DietCode shape (H = 2304), and on DietCode's BatchMatmulNT heads
    (192 x 120 x 120 x 64, full-size LDS tiles at T = 120); plus the causal
    scores of those heads (ragged T). Both arms run the register-ring engine
    (CAS_GEMM_F32=ring), the one kernel that has both forms; the default
    fp32 path (loads straight into LDS where that kernel applies, local
    padding only) is timed beside them as "default"."""
    import torch

    from causal_attention_score_amd import synth
    out = {}
    for name in ("dense_f32_960x1024x770", "dense_f32_960x2304x770", "bmm_nt_f32_192x120x120x64"):
        wl = synth.WORKLOADS[name]
        log(f"local-padding A/B on {name}")
        p = Part(wl)
        res = {}
        for variant in ("local_padding", "predicated", "default"):
            os.environ.pop("CAS_VARIANT", None)
            os.environ.pop("CAS_GEMM_F32", None)
            if variant != "default":
                os.environ["CAS_GEMM_F32"] = "ring"
            if variant == "predicated":
                os.environ["CAS_VARIANT"] = "predicated"
            _, (ms,), _, (md,), _ = time_parts([p], steps, 3, SUB_SETTLE_S)
            res[variant] = {"avg_launch_us": round(ms * 1e3, 2), "median_launch_us": round(md * 1e3, 2),
                            "useful_tflops": round(wl.useful_flops() / (ms * 1e-3) / 1e12, 2)}
        os.environ.pop("CAS_VARIANT", None)
        os.environ.pop("CAS_GEMM_F32", None)
        res["speedup"] = round(res["predicated"]["avg_launch_us"] / res["local_padding"]["avg_launch_us"], 3)
        if name.endswith("2304x770"):
            res["pages_context"] = ("DietCode on NVIDIA RTX: 0.98 vs 11.6 TFLOP/s (3090), 0.43 vs 5.27 (2080 Ti), "
                                    "baseline vs local padding; another machine, not a target")
        if name.startswith("bmm_nt"):
            res["pages_context"] = ("DietCode on NVIDIA RTX: 3.5 vs 8.7 TFLOP/s (3090), 1.8 vs 5.5 (2080 Ti), "
                                    "shrunk workspace vs local padding; another machine, not a target")
        out[name] = res
        del p
        torch.cuda.empty_cache()
    wl = synth.WORKLOADS["trimul_f32_B16_T120_NH12_HS64"]
    p = Part(wl)
    _, (ms,), _, (md,), _ = time_parts([p], steps, 3, SUB_SETTLE_S)
    out[wl.name] = {"avg_launch_us": round(ms * 1e3, 2), "median_launch_us": round(md * 1e3, 2),
                    "useful_tflops": round(wl.useful_flops() / (ms * 1e-3) / 1e12, 2),
                    "roofline": roofline_of(wl, ms)}
    del p
    torch.cuda.empty_cache()
    return out


def cpu_baseline(budget_s: float = 12.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of
    the workload: whole steps (the dense product, then the causal-score
    planes one (b, nh) plane at a time), repeated until the time budget is
    spent; a step cut short by the budget counts the planes it finished."""
    import oracle
    from causal_attention_score_amd import synth
    orc = oracle.get()
    wg = synth.WORKLOADS["dense_f32_960x1024x770"]
    wt = synth.WORKLOADS["trimul_f32_B8_T1024_NH12_HS64"]
    X, W = wg.inputs()
    (qkv,) = wt.inputs()
    B, T, NH, HS = wt.dims
    plane_flops = 2 * HS * T * (T + 1) // 2
    t0 = time.perf_counter()
    flops, steps, planes = 0, 0, 0
    while True:
        orc.gemm_nt(X, W, "f32", with_bound=False)
        flops += wg.useful_flops()
        for p in range(B * NH):
            b, h = divmod(p, NH)
            orc.trimul_causal_rows(qkv, B, T, NH * HS, NH, b, h, 0, T, "f32", with_bound=False)
            flops += plane_flops
            planes += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            steps += 1
            if time.perf_counter() - t0 <= budget_s:
                continue
        break
    dt = time.perf_counter() - t0
    part = planes - steps * B * NH
    step = f"dense fp32 960x1024x770 + {B * NH} causal-score planes (T={T}, HS={HS})"
    sample = f"{steps} whole steps of the workload ({step})" if steps else "part of one step"
    if part:
        sample += f"{' and' if steps else ':'} the dense product + {part} of {B * NH} planes"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2), "sample": sample + ", fp64 accumulation"}


def traffic_probe(names=PROBED) -> None:
    """Kernels for the rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE,
    then the SQ/GRBM busy counters, each a run of its own): one plain copy of
    512 MiB, whose counters calibrate the byte scale, then three launches of
    the kernel of each named workload, in the order given."""
    import torch

    from causal_attention_score_amd import synth
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for name in names:
        log(f"probe: 3 launches on {name}")
        p = Part(synth.WORKLOADS[name])
        for _ in range(3):
            p()
        torch.cuda.synchronize()
        del p
        torch.cuda.empty_cache()
    print("traffic probe done", flush=True)


def attention_probe() -> None:
    """Kernels for rocprofv3 counter runs of the attention kernels: three
    launches of the single-pass attention, then three of the attention from
    given statistics, on the 16-bit score workload (bf16 B4 T4096 NH25 HS64)."""
    import torch

    import causal_attention_score_amd as cas
    from causal_attention_score_amd import synth
    wl = synth.WORKLOADS["trimul_bf16_B4_T4096_NH25_HS64"]
    (qkv,) = wl.inputs()
    B, T, NH, HS = wl.dims
    q = device_tensor(qkv, wl.dtype)
    y = torch.empty((B, T, NH * HS), dtype=torch.float32, device="cuda")
    mx = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
    ls = torch.empty_like(mx)
    log("probe: 3 single-pass attention launches, then 3 from the statistics")
    for _ in range(3):
        cas.causal_attention_fused(q, NH, y=y, row_max=mx, row_logsum=ls)
    for _ in range(3):
        cas.causal_attention(q, NH, y=y, stats=(mx, ls))
    torch.cuda.synchronize()
    print("attention probe done", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-ab", action="store_true", help="skip the local-padding A/B")
    ap.add_argument("--no-softmax", action="store_true", help="skip the causal-softmax timings")
    ap.add_argument("--traffic-probe", nargs="*", metavar="WORKLOAD",
                    help="only launch the kernels for the rocprofv3 counter runs (default: every profiled workload)")
    ap.add_argument("--attention-probe", action="store_true",
                    help="only launch the 16-bit attention kernels for the rocprofv3 counter runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the hot path shards with no communication, "
              "so one GPU's share is what is measured; --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from causal_attention_score_amd import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.traffic_probe is not None:
        traffic_probe(tuple(args.traffic_probe) or PROBED)
        return
    if args.attention_probe:
        attention_probe()
        return
    wg = synth.WORKLOADS["dense_f32_960x1024x770"]
    wt = synth.WORKLOADS["trimul_f32_B8_T1024_NH12_HS64"]
    log("preparing inputs")
    parts = [Part(wg), Part(wt)]
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps (at least {SETTLE_S} s of them)")
    ms_step, per, wall_ms, med, warm_done = time_parts(parts, args.steps, args.warmup, SETTLE_S)
    flops = wg.useful_flops() + wt.useful_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    dom = max(range(2), key=lambda i: per[i])
    dom_wl = [wg, wt][dom]
    roof = roofline_of(dom_wl, per[dom], read_counters(dom_wl.name))
    parts_report = {wl.name: {"avg_launch_us": round(ms * 1e3, 2), "median_launch_us": round(md * 1e3, 2),
                              "useful_tflops": round(wl.useful_flops() / (ms * 1e-3) / 1e12, 2),
                              "roofline": roofline_of(wl, ms, read_counters(wl.name))}
                    for wl, ms, md in zip([wg, wt], per, med)}
    del parts
    torch.cuda.empty_cache()

    bf16 = None
    if not args.no_bf16:
        bf16 = {}
        # The two large shapes with 16-bit inputs; the scores also with 16-bit
        # outputs (the fp32 scores rounded once more: half the bytes written).
        for name, out in (("dense_bf16_4096", "f32"), ("trimul_bf16_B4_T4096_NH25_HS64", "f32"),
                          ("trimul_bf16_B4_T4096_NH25_HS64", "bf16"), ("dense_f16_4096", "f32"),
                          ("trimul_f16_B4_T4096_NH25_HS64", "f32"), ("trimul_f16_B4_T4096_NH25_HS64", "f16")):
            wl = synth.WORKLOADS[name]
            key = name if out == "f32" else f"{name}_out_{out}"
            log(f"timing {key}")
            p = Part(wl, out)
            _, (ms,), _, (md,), _ = time_parts([p], max(5, args.steps // 5), 2, SUB_SETTLE_S)
            bf16[key] = {"avg_launch_us": round(ms * 1e3, 2), "median_launch_us": round(md * 1e3, 2), "out_dtype": out,
                         "useful_tflops": round(wl.useful_flops() / (ms * 1e-3) / 1e12, 2),
                         "roofline": roofline_of(wl, ms, read_counters(name) if out == "f32" and name in KERNEL_SOURCES
                                                 else None, 4 if out == "f32" else 2)}
            del p
            torch.cuda.empty_cache()

    smx = None
    if not args.no_softmax:
        smx = softmax_timings(args.steps)

    ab = None
    if not args.no_ab:
        ab = local_padding_ab(max(10, args.steps // 2))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores")
        cpu = cpu_baseline()

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm_done, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) inputs of the pages' shapes)",
        "config": {"workload": "dense fp32 960x1024x770 + causal scores fp32 B=8 T=1024 NH=12 HS=64",
                   "gemm_nt": {"M": 960, "N": 1024, "K": 770, "dtype": "f32"},
                   "trimul_causal": {"B": 8, "T": 1024, "NH": 12, "HS": 64, "dtype": "f32"}},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parts": parts_report,
        "bf16_workloads": bf16,
        "causal_softmax": smx,
        "local_padding_ab": ab,
        "wall_ms_per_step": round(wall_ms, 5),
        "device": torch.cuda.get_device_name(0),
        # the seeded input streams (numpy PCG64) are not guaranteed stable across numpy versions
        "numpy": np.__version__,
        "sources_digest": {k: kernel_sources_digest(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
