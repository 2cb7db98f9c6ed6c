"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU, no
GPU): the fp64 oracle built with g++ -fsanitize=address,undefined runs the
oracle pins, and the C ABI's host code (argument validation, workspace and
cache layouts) built with the same sanitizers on the host side only runs the
ABI tests. Any sanitizer report aborts the child process and fails the
test. Device code is built as usual (no GPU sanitizer)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_child(tests, env_extra, tmp):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    lib = str(tmp_path / "liblocks_oracle_san.so")
    subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", lib, os.path.join(ROOT, "oracle", "locks_oracle.cpp")])
    out = _run_child(["tests/test_oracle_pins.py"], {"LOCKS_ORACLE_LIB": lib, "LD_PRELOAD": asan}, tmp_path)
    assert "passed" in out


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang ASan runtime not available")
    from sparse_kv_page_amd import build as B
    objs = [os.path.join(B.BUILD_DIR, s + ".o") for s in B.SOURCES if not s.endswith(".cpp")]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = str(tmp_path / "locks_api_san.o")
    # host code only carries the sanitizers (each -fsanitize behind -Xarch_host)
    subprocess.check_call([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-fno-gpu-rdc",
                           "-I" + os.path.join(ROOT, "include"), "-x", "hip", "-c",
                           os.path.join(B.CSRC, "locks_api.cpp"), "-o", api_o,
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"],
                          stderr=subprocess.DEVNULL)
    lib = str(tmp_path / "liblocks_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, api_o] + objs,
                          stderr=subprocess.DEVNULL)
    out = _run_child(["tests/test_abi.py"], {"LOCKS_LIB": lib, "LD_PRELOAD": rt[-1]}, tmp_path)
    assert "passed" in out
