"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU code (no GPU
needed): the oracle (plain C, built with gcc) and the library's host code
(every .hip source with the sanitizers on the host side only, linked with a
driver that exercises validation, workspace sizing, the capacity helper, the
error paths of every entry point and the 4-bit layout converter). Each driver
exits 0 only if every call returned the expected status; a sanitizer report
aborts it."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
# sanitizers on the host pass only (the device code is built as usual)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV_RUN = {"UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout,
                       env={**os.environ, **(env or {})})
    return r.returncode, r.stdout + r.stderr


def _check_clean(rc, out, what):
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "ERROR: LeakSanitizer" not in out, out[-4000:]
    assert rc == 0, f"{what} exited {rc}:\n{out[-4000:]}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wno-unknown-pragmas",
                    os.path.join(ROOT, "oracle", "moe_oracle.c"),
                    os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env={**ENV_RUN, "ASAN_OPTIONS": "detect_leaks=1"})
    _check_clean(rc, out, "oracle driver")
    assert "all calls ok" in out


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG),
                    reason="hipcc / ROCm clang++ not found")
def test_library_host_code_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "sparse_mixture_experts_40_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(SAN, "host_driver.cpp"))
    objs, procs = [], []
    for s in srcs:  # one compiler process per source, in parallel
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen(
            ["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
             "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for s, p in zip(srcs, procs):
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, f"{os.path.basename(s)}:\n{out[-4000:]}"
    exe = str(tmp_path / "host_driver")
    rc, out = _run([CLANG, "-fsanitize=address,undefined", *objs,
                    "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    assert rc == 0, out
    # leaks are not checked here: the HIP runtime keeps its own allocations to exit
    rc, out = _run([exe], env={**ENV_RUN, "ASAN_OPTIONS": "detect_leaks=0"})
    _check_clean(rc, out, "host driver")
    assert "all checks ok" in out
