"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only).

Two instrumented builds, each run in a process of its own under its
compiler's sanitizer runtime:
* libgdn.so with its host code (validation, workspace layout, launch plans,
  the graph cache and the per-device state behind its lock) instrumented
  and its device code built as usual; the C-ABI tests then run against it.
* the C oracle, built by gcc with the same two sanitizers; its pins then run
  against it.
Leak detection is off (the Python interpreter keeps its allocations at
exit); every other report aborts the run.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_token_fwd_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# each sanitizer flag right after -Xarch_host: host code only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def clang_asan_runtime() -> str:
    res = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        path = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
    return path


def gcc_asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_library(out: str) -> None:
    srcs = [os.path.join(CSRC, f) for f in ("gdn_api.hip", "gdn_proj.hip", "gdn_bwd.hip")]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", *HOST_SAN,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", out, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized hipcc build failed:\n{res.stderr[-4000:]}")


def build_oracle(out: str) -> None:
    cmd = ["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", out,
           os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)


def run(cmd, preload: str, extra_env: dict) -> subprocess.CompletedProcess:
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


ORACLE_PINS = """
import sys
import oracle
from tests import oracle_pins
orc = oracle.Oracle(sys.argv[1])
for pin in oracle_pins.ALL_PINS:
    pin(orc)
print("pins", len(oracle_pins.ALL_PINS))
"""


def run_library_tests(lib: str) -> subprocess.CompletedProcess:
    return run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                "tests/test_abi.py", "tests/test_binding_checks.py"], clang_asan_runtime(), {"GDN_LIBRARY": lib})


def run_oracle_pins(lib: str) -> subprocess.CompletedProcess:
    return run([sys.executable, "-c", ORACLE_PINS, lib], gcc_asan_runtime(), {})
