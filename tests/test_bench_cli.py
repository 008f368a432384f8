"""bench.py's command-line contract on a host without a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ, **(env or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=e, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr
    r = _run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_traffic_record_is_for_the_dense_kernel():
    """The committed counter record names the dense kernel and its per-launch bytes; bench.py
    reports it only while the kernel source hash matches."""
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert "fmha_bf16_kernel<false, false>" in rec["kernel"]
    assert rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] > 0
    t = bench.traffic_for_current_kernel()
    assert t is None or t == rec["hbm_bytes_per_launch"]
