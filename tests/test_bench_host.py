"""Host-side checks of bench.py (no GPU): more than one GPU is refused before
anything touches a device, the measured HBM traffic is reported only for the
kernel sources it was taken on, and every committed profile summary names the
rocprofv3 command that produced it."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

# route-kernel algorithmic bytes per launch, DeepSeek-V3-like: T (E*2 + k*4 + k*4) + E*4
ALG_BYTES = 16384 * (256 * 2 + 8 * 4 + 8 * 4) + 256 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                                 # no JSON line


def test_traffic_only_for_the_profiled_sources(monkeypatch):
    # the measured traffic is reported only while the route-kernel sources hash
    # to the ones the counters were taken on (else null); then the scaled
    # traffic is close to the algorithmic bytes (counting rows and bias reads
    # on top), never below them
    assert ALG_BYTES == 9438208
    path = os.path.join(ROOT, "profiles", "route_kernel_deepseek_v3_like_traffic.md")
    taken_on = None
    for line in open(path):
        if line.startswith("- source_sha256:"):
            taken_on = line.split(":", 1)[1].strip().strip("`")
    assert taken_on and len(taken_on) == 64
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: taken_on)
    v = bench.load_traffic("deepseek_v3_like")
    assert isinstance(v, int)
    assert ALG_BYTES <= v <= 1.25 * ALG_BYTES
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0" * 64)
    assert bench.load_traffic("deepseek_v3_like") is None
    assert bench.load_traffic("no_such_workload") is None


def test_profiles_name_their_commands():
    d = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(d))
    assert "route_permute_deepseek_v3_like_kernel_trace.md" in names
    assert "route_kernel_deepseek_v3_like_traffic.md" in names
    for n in names:
        text = open(os.path.join(d, n)).read()
        assert "rocprofv3 " in text, n
