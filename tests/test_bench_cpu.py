"""Host-side checks of the benchmark's command-line contract (no GPU is touched)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_one_json_line():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    msg = json.loads(lines[0])
    assert msg["n_gpus_requested"] == 2 and "one GPU" in msg["error"]


def test_help_lists_the_side_reports():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload-cfg", "--absorb-cfg", "--attn-only-cfg",
                 "--gram-only-cfg", "--steady", "--fp8", "--tempcache", "--future", "--no-cpu-baseline"):
        assert flag in r.stdout, flag
