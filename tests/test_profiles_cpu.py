"""The committed rocprofv3 summaries describe the committed kernels and workloads.

Each ``profiles/decode_<workload>_traffic.json`` (what ``bench.py`` reports as
``roofline.traffic``) must name a decode kernel, carry the hash of that kernel's current
source files, price the same algorithmic bytes the workload defines, and add up; each
kernel-statistics summary must cite the current hash of its kernel.  A kernel change
without a new profile fails here (the benchmark would report its traffic as null)."""
import glob
import json
import os
import re
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (no GPU needed: the helpers below touch no device)

TRAFFIC = sorted(glob.glob(os.path.join(ROOT, "profiles", "decode_*_traffic.json")))
STATS = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_kernel_stats.md")))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def test_every_benchmark_workload_has_a_traffic_summary():
    names = {os.path.basename(p)[len("decode_"):-len("_traffic.json")] for p in TRAFFIC}
    assert set(bench.SECONDARY) | set(bench.NEXT) | {"long"} <= names


@pytest.mark.parametrize("path", TRAFFIC, ids=[os.path.basename(p) for p in TRAFFIC])
def test_traffic_summary_matches_sources_and_workload(path):
    d = json.load(open(path))
    name = os.path.basename(path)[len("decode_"):-len("_traffic.json")]
    assert d["workload"] == name
    assert d["kernel"] in bench.KERNEL_FILES
    assert d["kernel_source_hash"] == bench.kernel_source_hash(d["kernel"]), \
        f"{name}: {d['kernel']} changed since its counters were taken; re-profile it"
    w = bench.make_workload(name)
    assert d["algorithmic_bytes_per_launch"] == int(np.sum(w.context_lens.astype(np.int64))) * w.kv_bytes_per_token()
    fetch = d["fetch_size_kib_per_dispatch"] * 1024 * d["fetch_scale"]
    write = d["write_size_kib_per_dispatch"] * 1024 * d["write_scale"]
    assert abs(d["hbm_bytes_per_launch"] - (fetch + write)) <= 1e-6 * d["hbm_bytes_per_launch"]
    # the copy calibration: a 2 GiB copy reads and writes 2 GiB
    assert d["copy_fetch_size_kib"] * d["fetch_scale"] == pytest.approx(d["copy_bytes_each_way"] / 1024)
    assert d["copy_write_size_kib"] * d["write_scale"] == pytest.approx(d["copy_bytes_each_way"] / 1024)
    assert 0.9 < d["fetch_over_algorithmic"] < 10


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_summaries_cite_the_current_sources(path):
    """Every summary gives its command and the hash of the kernel sources it was taken
    of (for a comparison of versions, the current one), which must be today's."""
    text = open(path).read()
    kernel = next(k for k in bench.KERNEL_FILES if os.path.basename(path).startswith(k))
    assert "rocprofv3 " in text and "bench.py" in text, f"{path}: no command"
    hashes = re.findall(r"(?:C|c)urrent kernel sources[^`]*`([0-9a-f]{16})`|Kernel sources[^`]*`([0-9a-f]{16})`", text)
    found = [a or b for a, b in hashes]
    assert found, f"{path}: no source hash"
    assert found[0] == bench.kernel_source_hash(kernel), f"{path}: stale summary; re-profile it"


@pytest.mark.parametrize("path", STATS, ids=[os.path.basename(p) for p in STATS])
def test_kernel_statistics_have_the_kernel_row(path):
    text = open(path).read()
    kernel = next(k for k in bench.KERNEL_FILES if os.path.basename(path).startswith(k))
    assert re.search(rf"^\| {kernel} \| \d+ \| \d+ \|", text, re.M), f"{path}: no row for {kernel}"
