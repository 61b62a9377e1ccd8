"""The library's host C++ (tree builder, batched builder, budget policy, argument checks and
split plans of every entry point) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer, and the CPU-tier host tests re-run against that build.

The kernel launchers are replaced by stand-ins that report no device, and the
no-allocation entry point by one that runs its checks and size limit without the device
array (tests/sanitize_stubs.cpp).  Any sanitizer report aborts the child run, which fails
this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_attention_draft_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HOST_SOURCES = ["api.cpp", "tree_meta.cpp", "budget.cpp"]
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_budget_host.py",
              "tests/test_batch_builder_host.py"]


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                    reason="needs g++ with the AddressSanitizer runtime")
def test_host_code_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    so = os.path.join(OUT, "libtreeverify_sanitized.so")
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "sanitize_stubs.cpp"))
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + [
           "-L", "/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["TV_SANITIZED_LIB"] = so
    child = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
             "-m", "not gpu", "-k", "not exports_every_declared"] + HOST_TESTS
    r = subprocess.run(child, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail, tail
    assert "runtime error" not in tail, tail
