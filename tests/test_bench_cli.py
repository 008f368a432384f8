"""bench.py's command-line contract on a host without a GPU."""
import json
import os
import subprocess
import sys

import pytest

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


def test_probe_library_exports_and_validates_before_any_device_call():
    """The benchmark's probe library (MFMA peak, instruction issue) exports its
    entry points, and the issue probe rejects bad arguments on the host."""
    import ctypes
    import subprocess
    path = os.path.join(ROOT, "diffusion_transformer_attention_non_amd", "libditattn_probe.so")
    if not os.path.exists(path):
        pytest.skip("libditattn_probe.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in ("mfma_probe_launch", "mfma_probe_flops_per_mfma", "mfma_probe_wall_rate_khz", "issue_probe_launch",
                 "issue_probe_per_iter", "issue_probe_valu_kinds", "issue_probe_coexec_modes"):
        assert name in exported, name
    lib = ctypes.CDLL(path)
    lib.issue_probe_launch.restype = ctypes.c_int
    lib.issue_probe_launch.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    dummy = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation first
    assert lib.issue_probe_valu_kinds() == 6 and lib.issue_probe_coexec_modes() == 5
    assert lib.issue_probe_per_iter(0) == 32 and lib.issue_probe_per_iter(1) == 4
    for args in ((2, 0, 1, 1, 1), (0, 6, 1, 1, 1), (1, 5, 1, 1, 1), (0, 0, 4, 1, 1), (0, 0, 0, 1, 1),
                 (1, 1, 3, 1, 1), (0, 0, 1, 0, 1), (0, 0, 1, 1, 0)):
        assert lib.issue_probe_launch(*args, dummy, dummy, None) == -1, args
    assert lib.issue_probe_launch(0, 0, 1, 1, 1, None, dummy, None) == -1
