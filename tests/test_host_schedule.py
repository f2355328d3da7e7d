"""Host replay of the decode step's schedule: tests/host/sched_check.cpp,
built for the host with hipcc (no GPU), runs the queues and the event tensor
that the device prologue builds (the same functions, pmk_sched.h) for the
model shapes and batches 1..1024, and checks for deadlock, notify counts and
producer-before-consumer order, and that no two row tiles' split-K records
in use at once overlap. Injected faults (a dropped notify, a counter armed one
too high or too low) must each be reported, and one split-K region shared by
all stages must be reported where records of two stages meet."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("sched") / "sched_check")
    src = os.path.join(HERE, "host", "sched_check.cpp")
    subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", src, "-o", out], check=True,
                   capture_output=True, timeout=300)
    return out


def test_schedule_replays_without_deadlock_or_early_consumer(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.mark.parametrize("fault", ["drop", "plus", "minus", "kpart"])
def test_replay_reports_injected_faults(exe, fault):
    r = subprocess.run([exe, "--fault", fault], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
