"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the
algorithmic byte counts behind the roofline objects, the reduction of
rocprofv3 counter CSVs to per-call traffic, the gate that keeps counter
readings to the kernel sources they were taken on, and the probe fraction
rule."""
import csv
import importlib.util
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_algorithmic_bytes(bench):
    # per token-head: q, k, v, o at 256 B each in bf16, log alpha 512 B,
    # beta 4 B; 64 KiB of fp32 state per (sequence, head) for h_final, and
    # as much again when h0 is read
    assert bench.prefill_alg_bytes(8192, 32, 1) == 262144 * 1540 + 32 * 65536
    assert bench.prefill_alg_bytes(8192, 32, 1) == 405_798_912
    assert bench.prefill_alg_bytes(100, 2, 3, h0=True) == 200 * 1540 + 2 * 6 * 65536
    # fp32 I/O: 512 B for each of q, k, v, o
    assert bench.prefill_alg_bytes(64, 1, 1, io_bytes=4) == 64 * (4 * 512 + 512 + 4) + 65536


def _write_counters(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counter_rows_reduce_to_bytes_per_call(bench, tmp_path):
    # two calls of a windowed prefill (two windows each: two intra and two
    # carry dispatches per call), one calibration copy, an unrelated kernel;
    # each dispatch reports its counter in several instances (summed)
    rows = []
    for call in range(2):
        for win in range(2):
            i = 10 * call + 2 * win
            rows += [(i, "kda::intra_kernel<__bf16, false>", "FETCH_SIZE", 100.0),
                     (i, "kda::intra_kernel<__bf16, false>", "FETCH_SIZE", 50.0),
                     (i + 1, "kda::carry_kernel<__bf16, 1>", "FETCH_SIZE", 30.0),
                     (i + 1, "kda::carry_kernel<__bf16, 1>", "WRITE_SIZE", 7.0)]
    rows += [(90, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 4.0),
             (91, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 9.0),
             (92, "some_other_kernel", "FETCH_SIZE", 1e9)]
    _write_counters(tmp_path / "run" / "x_counter_collection.csv", rows)
    per = bench._pmc_per_call(str(tmp_path / "run"), "FETCH_SIZE", calls=2)
    assert per["intra"] == pytest.approx(2 * 150.0)    # per call: two windows of 150
    assert per["carry"] == pytest.approx(2 * 30.0)
    assert per["copy"] == pytest.approx(9.0)           # the largest copy dispatch
    assert per["_dispatches"] == {"intra": 4, "carry": 4, "copy": 2}
    assert "some_other_kernel" not in per and None not in per


def test_decode_rows_are_the_recurrent_kernel(bench):
    assert bench._kernel_key("kda::recurrent_fwd_kernel<__bf16, float, false, true, 32>") == "decode"
    assert bench._kernel_key("kda::chunk_map_kernel(int const*, int, long)") == "chunk_map"
    assert bench._kernel_key("unrelated") is None


def _profile(tmp_path, sha, fetch=1000.0, write=500.0):
    text = "\n".join([
        "# comment lines are skipped", "workload = bench_step", f"sources_sha256 = {sha}",
        "calls = 3", "copy_read_factor = 2.0", "copy_write_factor = 1.0",
        "intra_dispatches = 3", f"intra_fetch_KiB = {fetch}", f"intra_write_KiB = {write}",
        "carry_dispatches = 3", "carry_fetch_KiB = 10.0", "carry_write_KiB = 20.0"])
    (tmp_path / "hbm_traffic_bench_step.txt").write_text(text + "\n")


def test_traffic_is_scaled_and_gated_on_the_sources(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", tmp_path)
    _profile(tmp_path, bench.sources_hash())
    t = bench.load_traffic("bench_step")
    assert t["intra"] == pytest.approx((1000.0 * 2.0 + 500.0 * 1.0) * 1024)
    assert t["carry"] == pytest.approx((10.0 * 2.0 + 20.0) * 1024)
    assert bench.prefill_traffic(t) == pytest.approx(t["intra"] + t["carry"])
    _profile(tmp_path, "0" * 16)   # taken on other kernel sources
    assert bench.load_traffic("bench_step") == {}
    assert bench.prefill_traffic({}) is None
    assert bench.load_traffic("no_such_workload") == {}


def test_committed_traffic_profiles_match_the_kernel_sources(bench):
    """The counter summaries under profiles/ were taken on the kernel sources
    in this tree (bench.py reports traffic only then)."""
    for wl in ("bench_step", "long_T131072", "packed_16_sequences"):
        assert bench.load_traffic(wl), f"profiles/hbm_traffic_{wl}.txt is stale or missing"


def test_probe_fraction_only_where_the_probe_bounds_the_kernel(bench):
    roof = bench._hbm(6.0e9, 1000.0)   # 6 GB in 1 ms
    assert roof["achieved"] == pytest.approx(6000.0) and roof["frac"] == pytest.approx(0.75)
    assert roof["traffic"] is None and "traffic_ratio" not in roof
    a = bench._with_probe(dict(roof), {"copy": 6500.0}, "copy")
    assert a["frac_achievable"] == pytest.approx(6000.0 / 6500.0) and "exceeds_probe" not in a
    b = bench._with_probe(dict(roof), {"copy": 5000.0}, "copy")
    assert b.get("exceeds_probe") is True and "frac_achievable" not in b
    c = bench._with_probe(dict(roof), None, "copy")
    assert "probe" not in c
    r = bench._hbm(1.0e9, 1000.0, traffic=2.7e9)
    assert r["traffic_ratio"] == pytest.approx(2.7)
