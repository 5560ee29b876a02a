"""CPU-side checks of bench.py: it refuses more than one GPU before touching
one, its algorithmic byte and instruction counts for the S6 workloads are the
ones the rooflines divide by, and a committed counter summary taken on other
kernel sources is reported as unknown (null), not as a stale figure."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench
from mamba_s6_selective_amd.workloads import S6_WORKLOADS

ROOT = Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
    assert r.stdout == ""  # no record printed


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--no-cpu-baseline", "--s6-only",
                 "--no-extras"):
        assert flag in r.stdout


# (b, t, d) elements, algorithmic HBM bytes, (b, t, d, n) elements and VALU
# instructions per (b, t, d, n) besides the exponential: u, delta read and y
# written once (2 + 2 + 4 B with bf16 inputs, 4 + 4 + 4 with fp32), B and C
# once per (b, t), A and D once; 4 instructions per direction-step, 6 for the
# bidirectional pass sharing its discretization.
EXPECTED = {
    "s6-fwd-b16-L1024-d256-N16-f32": (4194304, 50331648 + 2097152 + 17408, 67108864, 4),
    "s6-fwd-b1-L65536-d1024-N16-bf16": (67108864, 536870912 + 4194304 + 69632, 1073741824, 4),
    "s6-bidir-b4-L8192-d1536-N16-bf16": (50331648, 402653184 + 2097152 + 104448, 805306368, 6),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_s6_algorithmic_counts(name):
    assert bench.s6_algorithmic(S6_WORKLOADS[name]) == EXPECTED[name]


def test_peaks():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert abs(bench.VALU_PEAK_T - 39.3216) < 1e-9   # 256 CUs x 64 lanes x 2.4 GHz
    assert bench.LINEAR_BYTES_PER_ELEM == 12


def test_profile_records_follow_the_kernel_source(tmp_path, monkeypatch):
    """A traffic or VALU record is used only if it was taken on the kernel
    sources as they are now (hash of the csrc files named by the record)."""
    monkeypatch.setattr(bench, "PROFILES", tmp_path)
    assert bench.load_traffic("linear_scan", "linear_scan.hip", "scan_common.h") is None
    good = bench.source_hash("linear_scan.hip", "scan_common.h")
    (tmp_path / "linear_scan_traffic.json").write_text(
        json.dumps({"bytes_per_launch": 123.0, "kernel_source_sha": good}))
    assert bench.load_traffic("linear_scan", "linear_scan.hip", "scan_common.h") == 123.0
    (tmp_path / "linear_scan_traffic.json").write_text(
        json.dumps({"bytes_per_launch": 123.0, "kernel_source_sha": "0" * 16}))
    assert bench.load_traffic("linear_scan", "linear_scan.hip", "scan_common.h") is None
    w = "s6-fwd-b16-L1024-d256-N16-f32"
    s6 = bench.source_hash("s6_scan.hip", "s6_internal.h")
    (tmp_path / "s6_traffic.json").write_text(
        json.dumps({w: {"bytes_per_launch": 7.0, "kernel_source_sha": s6}}))
    (tmp_path / "s6_valu.json").write_text(
        json.dumps({w: {"kernels": {"k": 1}, "kernel_source_sha": "f" * 16}}))
    assert bench.load_s6_traffic(w) == 7.0
    assert bench.load_s6_valu(w) is None            # taken on other sources
    assert bench.load_s6_traffic("s6-fwd-b1-L65536-d1024-N16-bf16") is None  # no record
