"""The host-side code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the fp64 oracle on small ragged cases, and the C ABI's argument
validation with every kernel launcher stubbed to abort (so an invalid call
that reached a launch would fail the test).  Both programs are built from
the committed sources into a temporary directory and must exit 0."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"


def _run(exe, env_extra=None):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(env_extra or {})
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True, capture_output=True, text=True)
    # libgomp keeps its thread pool alive at exit; that is not a leak of the oracle's
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm clang++ not found")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    r = subprocess.run([CLANGXX, "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN,
                        "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "attention_sdpa_amd", "csrc"),
                        os.path.join(ROOT, "attention_sdpa_amd", "csrc", "attn_abi.cpp"),
                        os.path.join(HERE, "abi_driver.cpp"),
                        "-L", "/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the HIP runtime library allocates for the process lifetime when loaded
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})
