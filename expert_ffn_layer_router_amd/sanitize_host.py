"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of ``libmoe.so``, and a run
of the host-only ABI tests (``tests/test_abi_host.py``: argument checks, workspace layout
arithmetic, status strings, no kernel launch) against it.

Only host code is instrumented: every sanitizer flag is passed through ``-Xarch_host``, and the
device code is compiled as usual. The library lands in ``_build/asan/``; the tests run in a
child Python with the sanitizer runtime preloaded (Python itself is not instrumented), with
leak detection off (the interpreter keeps its own allocations to the end) and every report
fatal.

Run as ``python -m expert_ffn_layer_router_amd.sanitize_host``; exits with the test run's
status.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

from .build_lib import ARCH, CSRC, INCLUDE, ROOT, _hipcc, sources

OUT = ROOT / "_build" / "asan"
LIB = OUT / "libmoe_asan.so"

_HOST_SAN = ["-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]
_FLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", str(INCLUDE), "-I", str(CSRC), *_HOST_SAN]


def runtime() -> Path:
    """The shared ASan runtime of the compiler hipcc drives (it also holds UBSan's handlers)."""
    clang = Path(_hipcc()).resolve().parent.parent / "llvm" / "bin" / "clang"
    if not clang.exists():
        clang = Path("/opt/rocm/llvm/bin/clang")
    r = subprocess.run([str(clang), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    p = Path(r.stdout.strip())
    if not p.is_file():
        raise RuntimeError(f"ASan runtime not found (clang printed {p})")
    return p


def _compile(src: Path) -> Path:
    obj = OUT / (src.stem + ".o")
    r = subprocess.run([_hipcc(), *_FLAGS, "-c", str(src), "-o", str(obj)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> Path:
    OUT.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(len(srcs), os.cpu_count() or 1, 8))) as ex:
        objs = list(ex.map(_compile, srcs))
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *_HOST_SAN[:4],
                        "-shared-libsan", "-o", str(LIB), *map(str, objs)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return LIB


_CHILD = """
import sys
from pathlib import Path
sys.path[:0] = [{root!r}, {tests!r}]
import expert_ffn_layer_router_amd.binding as B
B.LIB_PATH = Path({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", {test!r}]))
"""


def run_host_tests(lib: Path = LIB, timeout: float = 600) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["LD_PRELOAD"] = str(runtime())
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = _CHILD.format(root=str(ROOT), tests=str(ROOT / "tests"), lib=str(lib),
                         test=str(ROOT / "tests" / "test_abi_host.py"))
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                          text=True, timeout=timeout)


if __name__ == "__main__":
    build()
    r = run_host_tests()
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    sys.exit(r.returncode)
