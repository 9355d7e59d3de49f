"""The host-side C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only):
  * the fp64 oracle (fmha_oracle.c: pthread work queue, strided indexing)
    built with gcc -fsanitize=address,undefined, running every oracle pin;
  * the library's host layer (argument validation, planning, the workspace
    and scratch logic of fmha_api.hip) built host-only with the sanitizers,
    running every C-ABI test.
Each suite runs in a child process with the sanitizer runtime preloaded and
any report fatal; the child's exit status and output are checked."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_pytest(test_file, env_extra, tmp_path):
    env = dict(os.environ, **env_extra)
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", test_file)]
    res = subprocess.run(cmd, cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "fmha_oracle.c"), "-o", lib, "-lm", "-lpthread"],
                   check=True, capture_output=True)
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    _run_pytest("test_oracle.py", {"FMHA_ORACLE_LIB": lib, "LD_PRELOAD": asan,
                                   "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                                   "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}, tmp_path)


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        path = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    return None


def test_host_layer_abi_checks_under_asan_and_ubsan(tmp_path):
    from head_attention_fmha_amd.build import hipcc
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime")
    lib = str(tmp_path / "libfmha_hostsan.so")
    csrc = os.path.join(ROOT, "head_attention_fmha_amd", "csrc")
    # the whole library for gfx950, with every -fsanitize applied to the host
    # code only (the device code is built as usual; the CPU tests launch nothing)
    cmd = [hipcc(), "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-O1", "-g",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "fmha_api.hip"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    _run_pytest("test_abi.py", {"FMHA_LIBRARY": lib, "LD_PRELOAD": rt,
                                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}, tmp_path)
