"""The CPU tier again, against AddressSanitizer + UndefinedBehaviorSanitizer
builds of the library's host code (host.cpp) and of the oracle (oracle.c):
planning, argument checks, the schedule, the cost model, descriptor
validation and every oracle routine run with memory and UB checks.  CPU
only (no device code is launched)."""
import os
import subprocess
import sys

import pytest

import sanitized_build

HERE = os.path.dirname(os.path.abspath(__file__))
FILES = ["test_capi_host.py", "test_cost_model.py", "test_oracle.py", "test_checkers.py"]


def test_cpu_tier_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    libs = sanitized_build.build(str(tmp_path))
    log = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=libs["runtime"], LCMA_LIBRARY=libs["lcma"], ORACLE_LIBRARY=libs["oracle"],
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}",
               LD_LIBRARY_PATH="/opt/rocm/llvm/lib:" + os.environ.get("LD_LIBRARY_PATH", ""))
    r = subprocess.run([sys.executable, "-m", "pytest", *[os.path.join(HERE, f) for f in FILES], "-q", "-x",
                        "-m", "not gpu", "-p", "no:cacheprovider"], cwd=os.path.dirname(HERE), env=env,
                       capture_output=True, text=True, timeout=1200)
    reports = [open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path) if f.startswith("san.")]
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], "\n".join(reports)[:6000])
    assert " passed" in r.stdout
