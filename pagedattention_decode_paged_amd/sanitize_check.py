"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the C ABI.

Builds the library with the sanitizers on its host code only (each
``-fsanitize=`` right after ``-Xarch_host``; the GPU code is built as usual)
into ``_build/asan/``, then runs the CPU tests of the boundary and of the
host block allocator (``tests/test_abi.py``, ``tests/test_allocator.py``)
against that build in a child process with the ASan
runtime preloaded (Python itself is not instrumented, so leak checking is
off).  Exits with the test run's status; a sanitizer report aborts the run.

Usage: python pagedattention_decode_paged_amd/sanitize_check.py
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def main() -> int:
    sys.path.insert(0, PKG)
    import build as b                        # the package's own build recipe (sources, flags)
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in b.SOURCES:
        obj = os.path.join(OUT, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        flags = [f for f in b.COMMON if f != "-O3"] + ["-O1", "-g"]
        cmd = [HIPCC, *lang, *flags, *SAN, "-c", os.path.join(b.CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True)
        objs.append(obj)
    lib = os.path.join(OUT, "libpagedkv.so")
    subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *SAN, "-o", lib, *objs],
                   check=True)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        print("no ASan runtime found", file=sys.stderr)
        return 2
    env = dict(os.environ, PAGEDKV_LIBRARY=lib, LD_PRELOAD=rt[-1],
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_allocator.py")],
                       env=env, cwd=ROOT)
    print(f"sanitized C-ABI and allocator tests: exit {r.returncode} ({lib})")
    return r.returncode


if __name__ == "__main__":
    sys.exit(main())
