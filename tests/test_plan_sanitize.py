"""The work planner under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/plan_fuzz.cpp drives csrc/host/plan.cpp (host C++, no GPU code) over
seeded random batches -- empty and one-token sequences, long ones, every page
size and planner knob -- and checks each plan's coverage of rows and keys, its
partial rows and its persistent queues.  It is built here with g++ and the
sanitizers, so an out-of-bounds access, a use after free or an overflow in
the planner aborts the run.  A copy built with PLANT_MISTAKE damages each plan
and must be caught, which keeps the checker itself honest.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
           os.path.join(ROOT, "varlen_paged_kv_amd", "csrc", "host", "plan.cpp")]
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build(tmp, extra=()):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = os.path.join(tmp, "plan_fuzz")
    r = subprocess.run(["g++", *FLAGS, *extra, *SOURCES, "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="vpk_plan_fuzz_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_planner_under_sanitizers(workdir, seed):
    exe = os.path.join(workdir, "plan_fuzz")
    if not os.path.exists(exe):
        _build(workdir)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "400", str(seed)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "400 plans checked" in r.stdout


def test_checker_catches_a_damaged_plan(workdir):
    sub = os.path.join(workdir, "planted")
    os.makedirs(sub, exist_ok=True)
    exe = _build(sub, ["-DPLANT_MISTAKE"])
    r = subprocess.run([exe, "50"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, r.stdout + r.stderr
    assert "parts end at" in r.stderr or "part starts at" in r.stderr
