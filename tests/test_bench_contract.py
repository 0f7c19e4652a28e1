"""CPU checks of the benchmark script's contract: it refuses more than one GPU with a JSON
message before touching any device, and every counter-measured traffic figure it reports
belongs to the kernel sources as they stand (a figure whose source hash no longer matches
would be reported as null)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_measured_traffic_matches_the_current_kernel_sources():
    for group, t in bench.MEASURED_TRAFFIC.items():
        assert bench.source_sha256(t["src"]) == t["sha256"], (
            f"{group}: the counter figures were taken on other sources; rerun the FETCH_SIZE / "
            f"WRITE_SIZE passes and update MEASURED_TRAFFIC")
        for kind in t:
            if kind in ("src", "sha256"):
                continue
            assert bench.measured_traffic(group, kind) > 0, (group, kind)
