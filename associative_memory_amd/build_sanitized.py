"""Host-sanitizer build of libkata, for checks on the CPU.

The host code of the C ABI (argument validation, planning, workspace layout,
the scratch-array bookkeeping: api.cpp and plan.cpp) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer, every check fatal; the
device-code objects are those of the regular build under _build/, unchanged,
so no GPU code carries a sanitizer.  The result is a separate library,
_build/sanitize/libkata.so.  To use it, load the binding with KATA_LIBRARY
set to that path and the compiler's ASan runtime (asan_runtime()) preloaded:

    python -m associative_memory_amd.build_sanitized   # prints the two paths
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as _b

OUT = os.path.join(_b.BUILD, "sanitize")
LIB = os.path.join(OUT, "libkata.so")
HOST_SOURCES = ("api.cpp", "plan.cpp")

# Each sanitizer flag applies to the host pass only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The shared ASan runtime of the hipcc toolchain (to preload into Python)."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(_b.hipcc())), "..", "llvm")
    for root in (llvm, "/opt/rocm/llvm"):
        hits = sorted(glob.glob(os.path.join(root, "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return os.path.realpath(hits[-1])
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def device_objects():
    """Objects of the regular build for every source that is not host-only."""
    objs = []
    for src in _b.sources():
        name = os.path.basename(src)
        if name in HOST_SOURCES:
            continue
        obj = os.path.join(_b.BUILD, name + ".o")
        if not os.path.exists(obj):
            raise RuntimeError(f"{obj} missing: run the regular build first")
        objs.append(obj)
    return objs


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = device_objects()
    flags = [f for f in _b.COMMON if f != "-O3"] + ["-O1", "-g"]
    for name in HOST_SOURCES:
        src = os.path.join(_b.CSRC, name)
        obj = os.path.join(OUT, name + ".o")
        cmd = [_b.hipcc()] + flags + SANITIZE + ["-x", "hip", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
        objs.insert(0, obj)
    cmd = [_b.hipcc(), f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-o", LIB] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {LIB}")
    return LIB


def environment(lib: str) -> dict:
    """Environment for a child Python that loads `lib` under the sanitizers."""
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (" " + pre if pre else "")
    env["KATA_LIBRARY"] = lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    lib = build(verbose=True)
    print(f"KATA_LIBRARY={lib}")
    print(f"LD_PRELOAD={asan_runtime()}")
    sys.exit(0)
