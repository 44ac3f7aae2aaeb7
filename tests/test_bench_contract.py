"""Host-side checks of bench.py: the one-GPU guard, the byte counts the
roofline figures divide by, and the readers of the committed profile
summaries.  No GPU is touched."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_per_head_token():
    # bf16 rows of d = 128 are 256 bytes: the forward reads q, k, v and
    # writes o; the backward reads q, k, v, dO and writes dq, dk, dv
    row = 2 * 128
    assert bench.KERNEL_BYTES["fwd_seg"] == 4 * row
    assert bench.KERNEL_BYTES["fwd_sum"] == 2 * row and bench.KERNEL_BYTES["bwd_sum"] == 2 * row
    assert bench.KERNEL_BYTES["fwd_fold"] == 0 and bench.KERNEL_BYTES["bwd_fold"] == 0
    # 62 of the 64 backward launches of a step also carry another piece's sums
    assert bench.KERNEL_BYTES["bwd_seg"] == pytest.approx(7 * row + 2 * row * 62 / 64)
    # one fp32 128 x 128 record per 256-token segment is 256 bytes per head-token
    assert 128 * 128 * 4 / 256 == 256
    for k in bench.KERNEL_BYTES:
        assert bench.KERNEL_DESIGN_BYTES[k] >= bench.KERNEL_BYTES[k]
    # delta rule: fp32 beta and gate in, fp32 dbeta out
    assert bench.DELTA_BYTES == {"fwd": 4 * row + 8, "bwd": 7 * row + 12}


def test_profile_readers_parse_the_committed_summaries():
    txt = open(bench.TRAFFIC_FILE).read()
    m = re.search(r"bytes_per_launch_calibrated:\s*([0-9.eE+]+)", txt)
    assert m and float(m.group(1)) > 0
    if re.search(r"kernel_source_sha256_16:\s*(\w+)", txt).group(1) == bench.kernel_source_hash():
        assert bench.traffic_from_profile("bwd_seg", 65536) == pytest.approx(float(m.group(1)))
    else:
        # counters taken on other kernel code are not reported
        assert bench.traffic_from_profile("bwd_seg", 65536) is None
    for name in ("fwd_seg", "bwd_seg"):
        busy = bench.mfma_busy_from_profile(name)
        assert busy is None or 0.0 < busy < 100.0


def test_every_profile_summary_names_its_command():
    d = os.path.join(ROOT, "profiles")
    for f in os.listdir(d):
        txt = open(os.path.join(d, f)).read()
        assert "rocprofv3" in txt and "bench.py" in txt, f
        assert len(txt) < 16 * 1024, f
