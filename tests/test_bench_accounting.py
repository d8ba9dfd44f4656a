"""CPU checks of the benchmark's accounting: algorithmic FLOPs and bytes per workload, the
source-hash guard on recorded HBM traffic, and the single-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("name,flops", [
    ("tiny", 4 * 256 * 256 * 64),                         # non-causal: 4 B Hq Sq Skv d
    ("mha2k", 4 * 4 * 16 * 2048 * 2048 * 64 // 2),        # causal FLOPs count half
    ("mha8k", 4 * 2 * 32 * 8192 * 8192 * 128 // 2),
    ("gqa32k", 4 * 1 * 32 * 32768 * 32768 * 128 // 2),    # GQA: counted per query head
])
def test_forward_flops(name, flops):
    assert bench.fwd_flops(WORKLOADS[name]) == flops


def test_forward_bytes_long_prefill():
    # Q, K, V read once (128 MiB each), O written once (128 MiB), LSE fp32 (2 MiB)
    assert bench.fwd_bytes(WORKLOADS["mha8k"]) == 4 * 128 * 2**20 + 2 * 2**20


def test_decode_bytes():
    d = bench.decode_bytes(WORKLOADS["decode"])
    kv = 2 * 64 * 16384 * 8 * 128 * 2           # K and V caches, bf16, read once
    q = 64 * 32 * 128 * 2
    assert d["split_kernel"] == kv + q
    assert d["total"] == kv + q + q + 64 * 32 * 4   # + O bf16 and LSE fp32 written


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    """A recorded HBM-traffic figure is reported only while the kernel sources it was
    measured on are unchanged."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    good = {"kernel_source_hash": bench.kernel_source_hash("fwd"), "hbm_bytes_per_launch": 123}
    (tmp_path / "good.txt").write_text(json.dumps(good) + "\nnotes\n")
    stale = dict(good, kernel_source_hash="0" * 16)
    (tmp_path / "stale.txt").write_text(json.dumps(stale) + "\n")
    assert bench.measured_traffic("good.txt", "fwd") == 123
    assert bench.measured_traffic("stale.txt", "fwd") is None
    assert bench.measured_traffic("missing.txt", "fwd") is None


def test_committed_traffic_records_parse():
    """Every committed traffic record carries the fields the benchmark reads."""
    prof = os.path.join(ROOT, "profiles")
    for name in os.listdir(prof):
        if not name.endswith("_hbm_traffic.txt"):
            continue
        with open(os.path.join(prof, name)) as f:
            rec = json.loads(f.readline())
        assert isinstance(rec["hbm_bytes_per_launch"], int) and rec["hbm_bytes_per_launch"] > 0, name
        assert len(rec["kernel_source_hash"]) == 16, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _local_includes(path):
    """Quoted #include targets of a source file, followed through the headers it includes."""
    import re
    csrc = os.path.dirname(path)
    seen, todo = set(), [os.path.basename(path)]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            for m in re.finditer(r'^\s*#include\s+"([^"]+)"', f.read(), re.M):
                if os.path.exists(os.path.join(csrc, m.group(1))):
                    todo.append(m.group(1))
    return seen


@pytest.mark.parametrize("family", sorted(bench.KERNEL_SOURCES))
def test_source_hash_families_cover_their_headers(family):
    """Each family's hash covers every kernel-directory file its kernel sources include, so
    a header change always invalidates the traffic figures measured on the old code."""
    csrc = os.path.join(ROOT, "io_aware_exact_21_amd", "csrc")
    listed = set(bench.KERNEL_SOURCES[family])
    for src in (f for f in listed if f.endswith(".hip")):
        missing = _local_includes(os.path.join(csrc, src)) - listed
        assert not missing, (family, src, sorted(missing))
