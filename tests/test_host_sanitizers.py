"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp and plan.cpp (validation, planning, workspace layout) are rebuilt with
both sanitizers, every finding fatal, and the whole host ABI suite
(test_abi_host.py: every entry point, every error path, plans and workspace
sizes over the supported shapes) runs against that library in a child
process.  No GPU is needed: nothing there launches a kernel.
"""
import os
import shutil
import subprocess
import sys

import pytest

from associative_memory_amd import build as regular_build

TESTS = os.path.dirname(os.path.abspath(__file__))


def _prerequisites():
    try:
        regular_build.hipcc()
    except RuntimeError:
        return "hipcc not available"
    for src in regular_build.sources():
        name = os.path.basename(src)
        if name.endswith(".hip") and not os.path.exists(os.path.join(regular_build.BUILD, name + ".o")):
            return "regular build objects missing (run __graft_entry__.build())"
    return None


@pytest.mark.skipif(_prerequisites() is not None, reason=str(_prerequisites()))
def test_abi_host_suite_under_asan_and_ubsan():
    from associative_memory_amd import build_sanitized as bs

    lib = bs.build()
    env = bs.environment(lib)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
           os.path.join(TESTS, "test_abi_host.py")]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900,
                       cwd=os.path.dirname(TESTS))
    out = r.stdout + r.stderr
    probe = subprocess.run([sys.executable, "-c", "import associative_memory_amd as am; print(am.lib()._name)"],
                           env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert " passed" in r.stdout
    shutil.rmtree(bs.OUT, ignore_errors=True)
