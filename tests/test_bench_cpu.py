"""bench.py's host logic, without a GPU: the one-GPU contract, the lookup of the
committed HBM counters, and the kernel names it reports for each timed case."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_is_read_only_for_the_sources_it_was_taken_on():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        tab = json.load(f)
    ent = tab["bf16"]
    assert bench.load_traffic("bf16", ent["src_sha"]) == ent["bytes_per_launch"]
    assert bench.load_traffic("bf16", "0" * 16) is None
    assert bench.load_traffic("no_such_case", ent["src_sha"]) is None


def test_ffn_roofline_traffic_is_the_sum_of_its_two_kernels():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        tab = json.load(f)
    want = tab["moe_ffn_up"]["bytes_per_launch"] + tab["moe_ffn_down"]["bytes_per_launch"]
    r = {"per_launch_us": [1400.0, 1410.0], "wall_s": 2.9e-3, "flops": 2.2e12,
         "min_bytes": 3.4e9, "meta": {}}
    out = bench.summarize("moe_ffn", r, 2)
    if tab["moe_ffn_up"]["src_sha"] == bench.kernel_sources_sha():
        assert out["roofline"]["traffic"] == want
    else:
        assert out["roofline"]["traffic"] is None


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "block_scaled_precision_05_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.SOURCES["gemm"]:
        (csrc / name).write_text("int a; // one\n/* two */ int b;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_sources_sha("gemm")
    (csrc / "gemm_kernel.h").write_text("int a;   // changed comment\n\n/* other */  int b;\n")
    assert bench.kernel_sources_sha("gemm") == h0
    (csrc / "gemm_kernel.h").write_text("int a; int c;\n")
    assert bench.kernel_sources_sha("gemm") != h0


def _stages(kind, K):
    """K stages of 64 bytes per row, as the launcher counts them."""
    row_bytes = {"bf16": 2 * K, "fp8": K, "fp4": K // 2}[kind]
    return (row_bytes + 63) // 64


def _leading_dead(nk, ns, kind):
    """The launcher's rule: pad nk to whole rounds of U stages (U = 2*NS for an odd
    ring, else NS); the padding goes first, rounded down to even, except for FP8
    when it is under 2% of the loop."""
    u = 2 * ns if ns % 2 else ns
    koff = (u - nk % u) & ~1 if nk % u else 0
    return 0 if kind == "fp8" and koff * 50 <= nk + koff else koff


@pytest.mark.parametrize("case,kind,K", [
    ("bf16", "bf16", 16384), ("fp8", "fp8", 16384), ("fp4", "fp4", 16384),
    ("grouped", "fp8", 7168), ("grouped_bf16", "bf16", 7168), ("grouped_fp4", "fp4", 7168),
    ("masked", "fp8", 7168), ("moe_ffn", "fp8", 7168), ("moe_ffn", "fp8", 2048),
])
def test_reported_kernel_names_match_the_launch(case, kind, K):
    name = bench.KERNEL_NAME[case]
    args = [a.strip() for a in re.match(r"gemm_kernel<([^>]*)>", name).group(1).split(",")]
    kind_id, ns, koff = int(args[0]), int(args[6]), int(args[10])
    assert kind_id == {"bf16": 0, "fp8": 1, "fp4": 2}[kind]
    assert koff == _leading_dead(_stages(kind, K), ns, kind)


def test_headline_is_the_cold_median_and_warm_is_reported_beside():
    r = {"per_launch_us": [900.0, 1000.0, 1100.0], "wall_s": 4e-3,
         "warm_us": [700.0, 800.0, 750.0], "warm_wall_s": 2.3e-3,
         "flops": 1e12, "min_bytes": 4e8, "meta": {}}
    out = bench.summarize("bf16", r, 3)
    assert out["tflops"] == pytest.approx(1e12 / 1000e-6 / 1e12)
    assert out["ms_per_call"] == pytest.approx(1.0)
    assert out["warm"]["tflops"] == pytest.approx(1e12 / 750e-6 / 1e12)
    # the roofline takes the mean cold launch
    assert out["roofline"]["achieved"] == pytest.approx(1e12 / 1000e-6 / 1e12)
    assert out["roofline"]["frac"] == pytest.approx(out["roofline"]["achieved"] / 2500.0)
    assert out["roofline"]["bound"] == "mfma"
    assert out["roofline"]["hbm_frac"] == pytest.approx(4e8 / 1000e-6 / 8e12)


def test_roofline_bound_is_the_longer_of_flops_and_bytes_at_peak():
    # 1 TFLOP at 5 PF takes 200 us; 2 GB at 8 TB/s takes 250 us: bound by HBM
    r = {"per_launch_us": [1000.0, 1000.0], "wall_s": 2e-3, "flops": 1e12, "min_bytes": 2e9,
         "meta": {}}
    out = bench.summarize("grouped", r, 2)
    assert out["roofline"]["bound"] == "hbm"
    assert out["roofline"]["unit"] == "GB/s"
    assert out["roofline"]["achieved"] == pytest.approx(2e9 / 1000e-6 / 1e9)
    assert out["roofline"]["frac"] == pytest.approx(2e9 / 1000e-6 / 8e12)
    assert out["roofline"]["mfma_frac"] == pytest.approx(1e12 / 1000e-6 / 5e15)
    # the rate stays in flops
    assert out["tflops"] == pytest.approx(1e12 / 1000e-6 / 1e12)
    r["min_bytes"] = 1e9   # 125 us: bound by the matrix cores
    assert bench.summarize("grouped", r, 2)["roofline"]["bound"] == "mfma"


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4", "grouped"])
def test_cpu_sample_times_the_oracle_on_the_case_inputs(kind):
    from block_scaled_precision_05_amd import workloads
    if kind == "grouped":
        w = workloads.grouped(4, 256, 256, 7, device="cpu", counts=[40, 0, 300, 5])
    else:
        w = workloads.dense(kind, 64, 256, 256, 7, device="cpu")
    r = bench.cpu_sample(kind, w, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOPS" and r["value"] > 0
    assert r["cores"] >= 1 and "rows 0.." in r["sample"]
    if kind == "grouped":
        assert "expert 2 (300 rows)" in r["sample"]


def test_host_info_names_cores_and_model():
    h = bench.host_info()
    assert h["nproc"] >= 1 and h["usable_cpus"] >= 1


def test_sample_parity_counts_what_the_oracle_disagrees_with():
    """bench.py compares the GPU output with the oracle rows its CPU sample computed:
    an output equal to bf16(oracle) reads 0, a planted wrong element is counted."""
    import numpy as np
    import torch
    import oracle
    r = np.random.default_rng(3)
    M, N, K = 200, 160, 64
    A = (r.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    B = (r.standard_normal((N, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    fn = lambda rows, cols=None: oracle.gemm_bf16(A, B, rows=rows, cols=cols)
    norms = lambda rows, cols: (oracle.row_norms("bf16", A, rows=rows),
                                oracle.row_norms("bf16", B, rows=cols))
    full = oracle.bf16_rne(fn(np.arange(M)))
    D = torch.from_numpy(full.view(np.int16).copy()).view(torch.bfloat16)
    kept = [(np.arange(0, 16), fn(np.arange(0, 16))), (np.arange(16, 80), fn(np.arange(16, 80)))]
    rep = bench._sample_parity(D, kept, fn, norms, 0, M, N, True)
    assert rep["outputs"] == 80 * N + 128 * 128 and rep["over_1e-3"] == 0
    assert rep["max_normalised_error"] == 0.0
    bad = full.copy()
    bad[5, 7] ^= 0x4000                      # a large change in one output
    bad[M - 1, N - 1] ^= 0x4000              # and one in the last tile
    D = torch.from_numpy(bad.view(np.int16).copy()).view(torch.bfloat16)
    rep = bench._sample_parity(D, kept, fn, norms, 0, M, N, True)
    assert rep["over_1e-3"] == 2

