"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds the library's host preparation (svdq_prepare.cpp, svdq_fp6_layout.cpp)
and the C ABI's argument checking (svdq_abi.hip, host side only, with the
kernel launchers replaced by stand-ins from tests/sanitize/abi_stubs.cpp)
with ROCm's clang and both sanitizers, links the driver in
tests/sanitize/driver.cpp, and runs it: every host preparation on small
ragged shapes and every argument check of the device entry points.  Device
code is not built here; the sanitizers apply to host code only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a4_rank_corrected_svdq_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", *SAN,
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# the ROCm runtime is not instrumented; its process-lifetime allocations are
# not the library's
LSAN_SUPPRESSIONS = "leak:libamdhip64\nleak:libhsa-runtime64\nleak:libamd_comgr\n"


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG) or shutil.which("ld") is None:
        pytest.skip("ROCm clang not available")
    out = tmp_path_factory.mktemp("sanitize")
    units = [
        (os.path.join(CSRC, "svdq_prepare.cpp"), ["-mavx2", "-mfma"]),
        (os.path.join(CSRC, "svdq_fp6_layout.cpp"), []),
        (os.path.join(CSRC, "svdq_abi.hip"), ["-x", "hip", "--offload-host-only", "--rocm-path=/opt/rocm"]),
        (os.path.join(HERE, "abi_stubs.cpp"), []),
        (os.path.join(HERE, "driver.cpp"), []),
    ]
    objs = []
    for src, extra in units:
        obj = str(out / (os.path.basename(src) + ".o"))
        rc, log = _run([CLANG, *FLAGS, *extra, "-c", src, "-o", obj])
        assert rc == 0, log
        objs.append(obj)
    exe = str(out / "driver")
    rc, log = _run([CLANG, *SAN, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-lpthread",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, log
    supp = out / "lsan.supp"
    supp.write_text(LSAN_SUPPRESSIONS)
    return exe, str(supp)


def test_host_code_clean_under_asan_ubsan(driver):
    exe, supp = driver
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    rc, log = _run([exe], env=env, timeout=300)
    assert rc == 0 and "SANITIZE OK" in log, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
