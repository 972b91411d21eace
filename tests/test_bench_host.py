"""Host-side logic of bench.py (no GPU): the FLOP and byte counts its roofline
divides by, the single-GPU contract, and the rule that counter traffic is only
reported for the kernel sources it was measured on.

The expected counts are the workloads' own arithmetic written out here from
the attention definition (4*N^2*d FLOP per head, halved for a causal mask; Q,
K, V read once, O and LSE written once), not recomputed through bench.py."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


@pytest.mark.parametrize("name,flop", [
    ("single_head_fp32", 4 * 1 * 1 * 128 ** 2 * 64),
    ("encoder_padded_bf16", 4 * 8 * 16 * 512 ** 2 * 64),
    ("decoder_causal_bf16", 4 * 8 * 12 * 1024 ** 2 * 64 // 2),
    ("long_causal_bf16", 4 * 1 * 32 * 8192 ** 2 * 128 // 2),
    ("long_causal_fp8", 4 * 1 * 32 * 16384 ** 2 * 128 // 2),
])
def test_nominal_flop_counts(name, flop):
    assert W.SPECS[name].flops() == pytest.approx(flop, rel=0, abs=0.5)


def test_headline_algorithmic_bytes():
    # bf16 Q, K, V read once and O written once (2 bytes each), fp32 LSE
    n, h, d = 8192, 32, 128
    expected = 4 * 2 * h * n * d + 4 * h * n
    assert expected == 269_484_032
    assert bench.algorithmic_bytes(W.SPECS["long_causal_bf16"]) == expected


def test_fp8_algorithmic_bytes():
    # e4m3 Q, K, V (1 byte), bf16 O (2 bytes), fp32 LSE
    n, h, d = 16384, 32, 128
    assert bench.algorithmic_bytes(W.SPECS["long_causal_fp8"]) == (3 * 1 + 2) * h * n * d + 4 * h * n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_is_reported_only_for_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = prof / "fa_fwd_long_causal_bf16_hbm_counters.md"
    assert bench.measured_traffic("long_causal_bf16") is None  # no summary
    path.write_text("traffic_bytes_per_launch: 123456789\n"
                    f"kernel_sources_sha256_16: {bench.kernel_sha()}\n")
    assert bench.measured_traffic("long_causal_bf16") == 123456789.0
    path.write_text("traffic_bytes_per_launch: 123456789\nkernel_sources_sha256_16: 0000000000000000\n")
    assert bench.measured_traffic("long_causal_bf16") is None  # taken on other sources
    # any edit to a kernel source invalidates the summary
    path.write_text("traffic_bytes_per_launch: 123456789\n"
                    f"kernel_sources_sha256_16: {bench.kernel_sha()}\n")
    src = tmp_path / bench.KERNEL_SOURCES[0]
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.measured_traffic("long_causal_bf16") is None
