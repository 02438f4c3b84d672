"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    # the benchmark measures one rank's share on one GPU; --gpus 2 must exit
    # non-zero before touching a device, with one JSON line saying why
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "--gpus must be 1" in msg["error"]


def test_counter_table_names_existing_kernel_sources():
    # every counter entry points at source files that exist, so its SHA-256
    # gate can be evaluated, at the profile its figures come from, and names
    # a workload the benchmark runs
    sys.path.insert(0, ROOT)
    import bench
    for wl, t in bench.COUNTERS.items():
        assert wl in bench.WORKLOADS
        for f in t["files"]:
            assert os.path.exists(os.path.join(ROOT, f)), (wl, f)
        if "profile" in t:
            assert os.path.exists(os.path.join(ROOT, t["profile"])), (wl, t["profile"])
        if "fetch_kib" in t:
            assert t["fetch_factor"] > 0 and t["write_factor"] > 0
        if "mfma_util" in t:
            assert 0 < t["mfma_util"] <= 1
