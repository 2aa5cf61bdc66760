"""bench.py's host-side logic without a GPU: it refuses more than one GPU, its design
bytes use the library's own record size, and the committed HBM counter summary it
reports as `roofline.traffic` was taken on the current forward kernel source."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (the module's work runs only under __main__)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("K,V", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_record_bytes_is_the_library_record(K, V):
    """The workspace of the dense forward is the schedule plus HV x chunks records, so
    two value-head counts with the same slice width differ by exactly their records."""
    from gated_delta_rule_64_amd import _lib
    if not os.path.exists(_lib.library_path()):
        from gated_delta_rule_64_amd import build
        build.build()
    T, nc = 8192, 8192 // 64
    w32 = _lib.kda_chunk_fwd_workspace_bytes(1, T, 16, 32, K, V, 1, False)
    w16 = _lib.kda_chunk_fwd_workspace_bytes(1, T, 16, 16, K, V, 1, False)
    rec = (w32 - w16) // (16 * nc)
    assert (w32 - w16) % (16 * nc) == 0
    assert rec == (bench.record_bytes(K, V, 2) + 255) // 256 * 256


def test_committed_counters_match_the_forward_source():
    """profiles/hbm_traffic_c3.json is keyed to the forward kernels' source; a change to
    them without new counters would make the bench report traffic as null."""
    d = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic_c3.json")))
    assert d["source_hash"] == bench.source_hash()
    per = bench.traffic_from_profiles()
    assert per is not None and set(per) == {"intra", "scan"}
    # each kernel moves at least the method's share of the bytes: Stage 1+2 its inputs,
    # the scan o (headline workload: 268,959,744 and 67,108,864 B)
    assert per["intra"] >= 268959744 and per["scan"] >= 67108864
    assert 0.4 < d["calibration"]["fetch_factor"] <= 1.0 and 0.4 < d["calibration"]["write_factor"] <= 1.0


def test_percentiles_and_stats():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0]
    st = bench.stats(xs)
    assert st["median"] == 3.0 and st["n"] == 5 and st["mean"] == 3.0
    assert bench.pctl(xs, 0.0) == 1.0 and bench.pctl(xs, 1.0) == 5.0
    assert st["p10"] <= st["median"] <= st["p90"]
