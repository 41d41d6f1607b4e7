"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the
roofline divides by, the refusal of more than one GPU, and the summary of a
kernel trace."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_four_streams():
    # per token at d = 5120: R 40,960 + h 10,240 + pre/post/comb 96 for the
    # fused call; R 40,960 + x 10,240 + post/comb 80 + R' 40,960 for hc_post
    n, d = 65536, 5120
    fused, post = bench.algorithmic_bytes(n, d)
    weights = 24 * 4 * d * 4 + 27 * 4          # hc_fn, hc_scale, hc_base once per launch
    assert fused == n * 51_296 + weights
    assert post == n * 92_240


def test_algorithmic_bytes_other_stream_counts():
    n, d = 1000, 256
    for hc in (1, 2, 3, 5, 8):
        M = (2 + hc) * hc
        fused, post = bench.algorithmic_bytes(n, d, hc)
        assert fused == n * (2 * hc * d + 2 * d + 4 * (2 * hc + hc * hc)) + 4 * M * hc * d + 4 * (3 + M)
        assert post == n * (2 * hc * d + 2 * d + 4 * (hc + hc * hc) + 2 * hc * d)
    assert bench.algorithmic_bytes(n, d, 4) == bench.algorithmic_bytes(n, d)


def test_boundary_bytes():
    # one sublayer boundary reads x, R, post/comb once and writes R', h and
    # the next coefficients once: 102,576 B per token at d = 5120
    n, d = 64, 5120
    assert bench.boundary_bytes(n, d) == n * 102_576 + 24 * 4 * d * 4 + 27 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_source_hash() == h


def _write_trace(d, kernels):
    """A minimal rocprofv3 kernel_stats.csv / kernel_trace.csv pair."""
    with open(os.path.join(d, "kt_kernel_stats.csv"), "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_ALL)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        for name, durs in kernels.items():
            w.writerow([name, len(durs), sum(durs), sum(durs) / len(durs), 0, min(durs), max(durs), 0])
    with open(os.path.join(d, "kt_kernel_trace.csv"), "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_ALL)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, durs in kernels.items():
            for i, du in enumerate(durs):
                w.writerow([name, 1000 * i, 1000 * i + du])


def test_summarize_trace_general_stream_count(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    tdir = tmp_path / "trace"
    tdir.mkdir()
    # two warmup dispatches, then two timed ones of each kernel
    _write_trace(str(tdir), {
        "void hc::(anonymous namespace)::k_gmm<2, 128>(unsigned short const*, float const*, float*, float*, long, int, int, float)":
            [90_000, 90_000, 30_000, 30_000],
        "void hc::(anonymous namespace)::k_gred<2>(float const*, float*, long, float, float)":
            [10_000, 10_000, 10_000, 10_000],
        "void hc::(anonymous namespace)::k_gsplit<2>(float const*, float const*, float const*, float*, float*, float*, long, int, float)":
            [5_000, 5_000, 4_000, 4_000],
        "void hc::(anonymous namespace)::k_gpre<2>(unsigned short const*, float const*, unsigned short*, long, int)":
            [30_000, 30_000, 20_000, 20_000],
        "void hc::(anonymous namespace)::k_gpost<2>(unsigned short const*, unsigned short const*, float const*, float const*, unsigned short*, long, int)":
            [40_000, 40_000, 33_000, 33_000],
    })
    bench.summarize_trace(str(tdir), 4096, 5120, "cmd", warmup=2, steps=2, tag="hc2", hc=2)
    text = (tmp_path / "kernel_trace_hc2_n4096_d5120.md").read_text()
    assert "n=4096 tokens, d=5120, hc=2" in text
    assert "| k_gmm<2, 128> |" in text and "| k_gpost<2> |" in text
    fused, post = bench.algorithmic_bytes(4096, 5120, 2)
    row = [l for l in text.splitlines() if l.startswith("| k_gmm + k_gred + k_gsplit + k_gpre")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    # timed region: 30 + 10 + 4 + 20 us
    assert float(cells[7]) == pytest.approx(64.0)
    assert float(cells[8]) == pytest.approx(fused / 64e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=1e-3)
    prow = [l for l in text.splitlines() if l.startswith("| k_gpost<2> |")][0]
    pcells = [c.strip() for c in prow.strip("|").split("|")]
    assert float(pcells[7]) == pytest.approx(33.0)
    assert float(pcells[8]) == pytest.approx(post / 33e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=1e-3)


def _write_counters(d, counter, rows):
    os.makedirs(os.path.join(d, counter), exist_ok=True)
    with open(os.path.join(d, counter, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_ALL)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            w.writerow([i + 1, name, counter, v])


def test_summarize_counters_calibrates_on_the_one_gib_copy(tmp_path, monkeypatch):
    # the run copies a larger buffer too (a clone of the residual): the
    # calibration must take the 1 GiB copy, not the largest one
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    d = str(tmp_path / "pmc")
    copy = "__amd_rocclr_copyBuffer"
    spec = "void hc::spec::k_spec<5, true, false>(hc::CoopArgs)"
    post = "void hc::k_post<true>(HIP_vector_type<unsigned int, 4u> const*)"
    n, dd = 65536, 5120
    fb, pb = bench.algorithmic_bytes(n, dd)
    kib = 1 << 20                                   # KiB in 1 GiB
    # counters read as the real ones do: FETCH_SIZE half the bytes a copy
    # moves, WRITE_SIZE all of them
    _write_counters(d, "FETCH_SIZE", [(copy, 2.5 * kib / 2), (spec, 1.1 * fb / 2048), (post, pb / 2 / 2048),
                                      (copy, kib / 2)])
    _write_counters(d, "WRITE_SIZE", [(copy, 2.5 * kib), (spec, 0.1 * fb / 1024), (post, pb / 2 / 1024),
                                      (copy, kib)])
    bench.summarize_counters(d, n, dd, "cmd")
    text = (tmp_path / "hbm_traffic_n65536_d5120.md").read_text()
    assert "FETCH_SIZE read 524288 KiB" in text and "(x2.0000)" in text and "(x1.0000)" in text
    row = [l for l in text.splitlines() if l.startswith("| k_spec ")][0]
    assert float(row.strip("|").split("|")[-1]) == pytest.approx(1.2, abs=1e-3)
    prow = [l for l in text.splitlines() if l.startswith("| k_post ")][0]
    assert float(prow.strip("|").split("|")[-1]) == pytest.approx(1.0, abs=1e-3)
