"""Host-side logic of bench.py (CPU only): the launch groupings of a sweep,
the kernel family of each workload and the validity check of the stored
traffic figures."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gemm_tkq_gemv_amd import inputs  # noqa: E402


def _check_partition(groups, n):
    flat = [i for g in groups for i in g]
    assert sorted(flat) == list(range(n)) and flat == sorted(flat)   # every matrix once, in sweep order


def test_launch_groups_partition_the_sweep():
    for model, layers in (("qwen2.5-0.5b", 24), ("qwen2.5-7b", 28)):
        shapes = inputs.sweep_shapes(model)
        n = len(shapes)
        assert bench.launch_groups(shapes, "grouped") == [list(range(n))]
        per = bench.launch_groups(shapes, "per-matrix")
        assert len(per) == n
        _check_partition(per, n)
        staged = bench.launch_groups(shapes, "staged")
        _check_partition(staged, n)
        assert len(staged) == 4 * layers + 1
        names = [[shapes[i][0].split(".")[-1] for i in g] for g in staged]
        assert names[:4] == [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
        assert names[-1] == ["lm_head"]


def test_traffic_family():
    assert bench.traffic_family("0.5b-int4") == "gemv"
    assert bench.traffic_family("0.5b-int4-greedy") == "gemv"
    assert bench.traffic_family("7b-int4") == "gemv"
    assert bench.traffic_family("bin") == "gemv"
    assert bench.traffic_family("0.5b-int4-m16") == "small_m"
    assert bench.traffic_family("7b-int4-m16") == "small_m"
    assert bench.traffic_family("7b-prefill") == "prefill"
    assert bench.traffic_family("kv-32k-gqa") == "kv"


def test_stored_traffic_needs_matching_sources(monkeypatch):
    w = "0.5b-int4"
    fam, nbytes, h = bench.TRAFFIC_BYTES[w]
    assert fam == bench.traffic_family(w)
    monkeypatch.setitem(bench.TRAFFIC_BYTES, w, (fam, nbytes, "0" * 16))
    assert bench.measured_traffic(w) is None                  # sources changed since the profile
    monkeypatch.setitem(bench.TRAFFIC_BYTES, w, (fam, nbytes, bench.source_hash(fam)))
    assert bench.measured_traffic(w) == nbytes
    assert bench.measured_traffic("no-such-workload") is None
