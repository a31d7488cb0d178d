"""Host logic of bench.py, no GPU: the algorithmic work formulas on small cases
counted by hand, the traffic record lookup (reported only for its own kernel
and workload while the kernel sources still hash to the recorded value), and
the refusal of runs over several GPUs."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_dense_work_counts_every_operand_once():
    # M=3, N=130, K=256: A 3*256, alpha 3*2 floats, B 130*256, beta 2x2 floats, D 3*130 bf16
    flops, nbytes = bench.dense_work(3, 130, 256)
    assert flops == 2 * 3 * 130 * 256
    assert nbytes == 3 * 256 + 4 * 3 * 2 + 130 * 256 + 4 * 2 * 2 + 2 * 3 * 130


def test_grouped_work_skips_empty_groups():
    # experts with 0 (or a negative, clamped) row count read no weights and do no work
    f1, b1 = bench.grouped_work([5], 128, 128, 0)
    f2, b2 = bench.grouped_work([0, 5, -3], 128, 128, 12)
    assert f1 == f2 == 2 * 5 * 128 * 128
    assert b2 == b1 + 12
    assert b1 == 5 * 128 + 4 * 5 + 128 * 128 + 4 + 2 * 5 * 128


def test_kgrouped_work():
    # fp32 C read and D written for each of the 2 groups; flops over the valid tokens only
    flops, nbytes = bench.kgrouped_work(4, 8, [100, 28], 256)
    assert flops == 2 * 4 * 8 * 128
    assert nbytes == (4 + 8) * 256 + 4 * (4 + 8) * 2 + 8 * 2 * 4 * 8 + 4 * 2


def test_roof_time_takes_the_binding_limit():
    # 5e12 flops at 5 PF/s = 1000 us; 8e9 bytes at 8 TB/s = 1000 us
    assert bench.roof_time_us(5e12, 1.0) == pytest.approx(1000.0)
    assert bench.roof_time_us(1.0, 8e9) == pytest.approx(1000.0)
    assert bench.roof_time_us(5e12, 16e9) == pytest.approx(2000.0)


def _record(path, kernel, workload, sha, value):
    with open(path, "w") as f:
        f.write("# record\n\nsome text: not a field\n\n")
        f.write(f"- kernel: {kernel}\n- workload: {workload}\n- source_sha256: {sha}\n")
        f.write(f"- traffic_bytes_per_launch: {value}\n")


def test_recorded_traffic_only_for_its_kernel_workload_and_sources(tmp_path, monkeypatch):
    rec = tmp_path / "rec.md"
    monkeypatch.setattr(bench, "TRAFFIC_RECORDS", {"sweep": str(rec)})
    sha = bench.kernel_source_hash()
    _record(rec, "k", "sweep", sha, 123456)
    assert bench.recorded_traffic("k", "sweep") == 123456.0
    assert bench.recorded_traffic("other", "sweep") is None
    assert bench.recorded_traffic("k", "masked") is None          # no record for that workload
    _record(rec, "k", "sweep", "0" * 64, 123456)                   # sources changed since the record
    assert bench.recorded_traffic("k", "sweep") is None
    _record(rec, "k", "masked", sha, 123456)                       # record of another workload
    assert bench.recorded_traffic("k", "sweep") is None
    rec.unlink()
    assert bench.recorded_traffic("k", "sweep") is None            # missing record


def test_committed_records_name_their_workload():
    for workload, path in bench.TRAFFIC_RECORDS.items():
        with open(path) as f:
            text = f.read()
        assert f"- workload: {workload}\n" in text and "- traffic_bytes_per_launch: " in text


def test_several_gpus_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       env=env, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
