"""bench.py's host side, with no GPU: the refusal of more than one GPU, the
roofline entries against byte and FLOP counts worked out by hand from the
workload shapes, and the reading of committed counter summaries."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from causal_attention_score_amd import synth  # noqa: E402


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


# (workload, useful FLOPs, algorithmic bytes with fp32 output), each worked out
# from the shapes: dense 2MNK and es(MK + NK) + 4MN; scores 2 HS T(T+1)/2 per
# plane, Q and K read once, the whole (T, T) plane written.
COUNTS = [
    ("dense_f32_15x9x12", 2 * 15 * 9 * 12, 4 * (15 * 12 + 9 * 12) + 4 * 15 * 9),
    ("dense_f32_960x1024x770", 1_513_881_600, 10_042_880),
    ("trimul_f32_B8_T1024_NH12_HS64", 6_448_742_400, 452_984_832),
    ("dense_bf16_4096", 137_438_953_472, 134_217_728),
    ("trimul_bf16_B4_T4096_NH25_HS64", 107_400_396_800, 6_815_744_000),
]


@pytest.mark.parametrize("name,flops,nbytes", COUNTS, ids=[c[0] for c in COUNTS])
def test_workload_counts(name, flops, nbytes):
    wl = synth.WORKLOADS[name]
    assert wl.useful_flops() == flops
    assert wl.algorithmic_bytes() == nbytes


def test_scores_16bit_output_bytes():
    wl = synth.WORKLOADS["trimul_bf16_B4_T4096_NH25_HS64"]
    # Q and K in bf16 (2 bytes), the planes in 2-byte elements
    assert wl.algorithmic_bytes(2) == 2 * 2 * 4 * 4096 * 25 * 64 + 2 * 4 * 25 * 4096 * 4096


def test_roofline_scores_is_hbm_bound():
    wl = synth.WORKLOADS["trimul_f32_B8_T1024_NH12_HS64"]
    r = bench.roofline_of(wl, 0.1, None)  # 100 us per launch
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(452_984_832 / 100e-6 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, rel=1e-3)
    assert r["traffic"] is None
    r = bench.roofline_of(wl, 0.1, {"hbm_bytes_per_launch": 453_000_000.0, "mfma_busy_frac": 0.25})
    assert r["traffic"] == pytest.approx(4530.0, rel=1e-3)
    assert r["traffic_bytes_per_launch"] == 453_000_000
    assert r["traffic_over_algorithmic"] == pytest.approx(453_000_000 / 452_984_832, rel=1e-4)
    assert r["counters"] == {"mfma_busy_frac": 0.25}


@pytest.mark.parametrize("name,peak", [("dense_f32_960x1024x770", 157.3), ("dense_bf16_4096", 2516.6),
                                       ("dense_f16_4096", 2516.6)])
def test_roofline_dense_is_mfma_bound(name, peak):
    wl = synth.WORKLOADS[name]
    r = bench.roofline_of(wl, 0.02, None)  # 20 us per launch
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == peak
    assert r["achieved"] == pytest.approx(wl.useful_flops() / 20e-6 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / peak, rel=1e-3)


def test_sources_digest_is_stable():
    for k in bench.KERNEL_SOURCES:
        d = bench.kernel_sources_digest(k)
        assert len(d) == 16 and int(d, 16) >= 0
        assert d == bench.kernel_sources_digest(k)


def test_read_counters_only_for_matching_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "counters_k.md").write_text(
        "# summary\n\n- sources_digest: `0123456789abcdef`\n- hbm_bytes_per_launch: `453259002`\n"
        "- mfma_busy_frac: `0.57`\n- wait_frac: `n/a`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda k: "0123456789abcdef")
    assert bench.read_counters("k") == {"hbm_bytes_per_launch": 453259002.0, "mfma_busy_frac": 0.57}
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda k: "fedcba9876543210")
    assert bench.read_counters("k") is None
    assert bench.read_counters("missing") is None


def test_every_profiled_workload_is_a_workload():
    for k in bench.KERNEL_SOURCES:
        assert k in synth.WORKLOADS
