"""bench.py's paths that need no GPU: the one-GPU guard and the profiling
command lines (CPU, no device access)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "4")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profile_commands_are_complete():
    r = _run("--profile-commands", "OUT")
    assert r.returncode == 0
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 7
    for line in lines:
        assert line.startswith("timeout ") and " rocprofv3 " in line and " -- python3 bench.py" in line
        assert "-d OUT/" in line
    # counters in their own runs, never combined with tracing
    pmc = [l for l in lines if "--pmc" in l]
    assert len(pmc) == 6 and all("--kernel-trace" not in l for l in pmc)
    assert sum("--kernel-trace" in l for l in lines) == 1
    # one pass stays within the per-block counter limits: at most 8 SQ_, 4 TCC_ and 2 GRBM_
    for l in pmc:
        names = l.split("--pmc ")[1].split(" --")[0].split()
        assert sum(n.startswith("SQ_") for n in names) <= 8
        assert sum(n.startswith("GRBM_") for n in names) <= 2
        assert sum(n in ("FETCH_SIZE", "WRITE_SIZE") for n in names) <= 1
