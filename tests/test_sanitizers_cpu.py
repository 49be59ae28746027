"""Host-side sanitizers (CPU only, no GPU): the oracle's pins run against an oracle built with
gcc's AddressSanitizer and UBSan, and the C ABI's CPU tests (argument validation, status
codes, the launch-plan override, the allocation-free entry point's size check) run against
a library whose host code is built with clang's AddressSanitizer and UBSan.  Each suite runs
in a subprocess with the sanitizer runtime preloaded; any report aborts it."""
import glob
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
CSRC = ROOT / "selective_scan_ss2d_amd" / "csrc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(cmd):
    out = subprocess.run(cmd, capture_output=True, text=True).stdout.strip()
    return out if out and os.path.exists(out) else None


def _run_suite(test_file, preload, extra_env, selector=None):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           str(ROOT / "tests" / test_file)]
    if selector:
        cmd += ["-k", selector]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, (res.stdout[-3000:] + res.stderr[-3000:])
    assert "passed" in res.stdout


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    libasan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if libasan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared",
                    "-std=c11", str(ROOT / "oracle" / "ss2d_oracle.c"), "-o", str(lib), "-lm"],
                   check=True, capture_output=True, text=True)
    _run_suite("test_oracle_pins.py", libasan, {"SS2D_TEST_ORACLE_LIBRARY": str(lib)},
               "test_pin or golden or thread")


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not runtimes:
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    from selective_scan_ss2d_amd import build
    objs = [build.BUILD / (src.stem + ".o") for src in build.sources()
            if src.name != "ss2d_abi.hip"]
    if not all(o.exists() for o in objs):
        build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    abi = tmp_path / "ss2d_abi_san.o"
    flags = [f for f in build.COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([hipcc, *flags, *san, "-c", str(CSRC / "ss2d_abi.hip"), "-o", str(abi)],
                   check=True, capture_output=True, text=True)
    lib = tmp_path / "libss2d_san.so"
    subprocess.run([hipcc, f"--offload-arch={build.ARCH}", "-shared", "-fPIC", *san[:4],
                    str(abi), *map(str, objs), "-o", str(lib)],
                   check=True, capture_output=True, text=True)
    _run_suite("test_abi_cpu.py", runtimes[0], {"SS2D_TEST_LIBRARY": str(lib)})
