"""Host-side sanitizer runs (CPU only): the double-precision oracle built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer under its own pin tests, and the C ABI's
host code (argument validation, workspace layout, error reporting in spa_api.cpp) built with
clang's AddressSanitizer and UndefinedBehaviorSanitizer for the host pass only (the device
code is unchanged) under the ABI tests. Each run is a child Python process with the sanitizer
runtime preloaded (the interpreter itself is not instrumented); a sanitizer report or a
non-zero exit fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "jl_feature_projected_amd")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")


def _run_child(code: str, preload: str, timeout: int = 600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def _gcc_runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def test_oracle_under_asan_and_ubsan(tmp_path):
    import oracle

    lib = str(tmp_path / "libspa_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC",
                    "-shared", "-std=c11", "-Wall", "-Wextra", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", lib, oracle.SRC_PATH, "-lm"],
                   check=True)
    preload = _gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so")
    tests = ["tests/test_oracle_pins.py", "tests/test_oracle_bwd.py",
             "tests/test_oracle_decode.py", "tests/test_oracle_sfa.py",
             "tests/test_oracle_sparse_projection.py", "tests/test_oracle_mutants.py"]
    code = ("import sys, pytest, oracle\n"
            f"oracle.LIB_PATH = {lib!r}\n"
            f"sys.exit(pytest.main({tests!r} + ['-q', '-x', '-p', 'no:cacheprovider', "
            "'-m', 'not gpu']))\n")
    out = _run_child(code, preload)
    assert " passed" in out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    from jl_feature_projected_amd import build as B

    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
            if s != "spa_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = str(tmp_path / "spa_api_san.o")
    flags = [f for f in B.compile_flags() if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    # sanitizers for the host pass only (each -fsanitize= right after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    subprocess.run([B.hipcc(), *flags, *san, "-c", os.path.join(B.CSRC, "spa_api.cpp"), "-o",
                    api_o], check=True, capture_output=True)
    lib = str(tmp_path / "libspa_hostsan.so")
    subprocess.run([B.hipcc(), "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *san, "-o", lib,
                    api_o, *objs], check=True, capture_output=True)
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no clang ASan runtime")
    code = ("import sys, pytest\n"
            "import jl_feature_projected_amd as spa\n"
            f"spa.LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['tests/test_abi_cpu.py', '-q', '-x', '-p', "
            "'no:cacheprovider', '-m', 'not gpu']))\n")
    out = _run_child(code, rt[-1])
    assert " passed" in out
