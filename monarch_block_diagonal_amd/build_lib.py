"""Builds the Monarch HIP library in-tree: monarch_block_diagonal_amd/libmonarch.so.

Every source under csrc/ is compiled by hipcc for gfx950 (one object per
file, in parallel) and linked into one shared library exporting the C ABI of
include/monarch.h. Run as `python -m monarch_block_diagonal_amd.build_lib`.

`--sanitize` builds a second copy, _build_asan/libmonarch_asan.so, whose host
code is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(device code is built as usual), and `--sanitize --test` then runs the host
ABI tests (tests/test_abi.py: argument checks, planning, descriptions; no
kernel launch) against it with the sanitizer runtime preloaded, failing on
any report.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmonarch.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# host-side sanitizer build (device code is compiled as usual)
BUILD_ASAN = os.path.join(HERE, "_build_asan")
LIB_ASAN = os.path.join(BUILD_ASAN, "libmonarch_asan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    build_dir = BUILD_ASAN if sanitize else BUILD
    lib = LIB_ASAN if sanitize else LIB
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """The AddressSanitizer runtime of the toolchain that built the library."""
    out = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("AddressSanitizer runtime not found")
    return found[-1]


def test_sanitized() -> int:
    """tests/test_abi.py against the sanitizer build; returns pytest's status."""
    env = dict(os.environ)
    env["MONARCH_LIBRARY"] = LIB_ASAN
    env["LD_PRELOAD"] = sanitizer_runtime()
    # the interpreter itself is not instrumented: its allocations are not
    # tracked as leaks; any other report aborts the run
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
           "-p", "no:cacheprovider"]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    san = "--sanitize" in sys.argv[1:]
    print(build(sanitize=san))
    if san and "--test" in sys.argv[1:]:
        sys.exit(test_sanitized())
