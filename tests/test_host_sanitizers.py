"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer.

The host sources (argument validation and the C ABI in api.cpp, the work-list
scheduler, the NSP planner, the timing hooks) are compiled with g++ and
-fsanitize=address,undefined into a separate library, with the kernel
launchers replaced by stand-ins that report failure
(tests/host_asan/launch_stubs.cpp).  The CPU tests of the C ABI and the
planner then run against that library in a child process with the
sanitizer runtime preloaded; any report ends the child with an error.
The plan cache's eviction rule (plan_cache.h) has a unit test of its own
(tests/host_asan/plan_cache_test.cpp), built and run with the same
sanitizers.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_sequence_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HOST_SOURCES = ["api.cpp", "scheduler.cpp", "router.cpp", "profiler.cpp"]


def _tool(name):
    return shutil.which(name)


def _build():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libvarlen_sanitized.so")
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "host_asan", "launch_stubs.cpp"))
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, *srcs, "-L/opt/rocm/lib", "-lamdhip64", "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return lib


@pytest.mark.timeout(600)
def test_host_code_under_address_and_ub_sanitizers():
    if not _tool("g++") or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs g++ and the ROCm runtime library")
    lib = _build()
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.exists(asan), "g++ has no AddressSanitizer runtime"
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    log = os.path.join(OUT, "report")
    for f in os.listdir(OUT):
        if f.startswith("report"):
            os.remove(os.path.join(OUT, f))
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:abort_on_error=1:log_path={log}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}"
    env["HIP_VISIBLE_DEVICES"] = ""
    # torch is not loaded in the child: the tests below that need it are
    # deselected (they check the Python binding, not the host code)
    code = (
        "import sys, pytest\n"
        f"sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        "import variable_length_sequence_amd as vl\n"
        f"vl.LIB_PATH = {lib!r}\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', '-k',\n"
        "    'not binding and not export', "
        f"{os.path.join(ROOT, 'tests', 'test_host_boundary.py')!r}, "
        f"{os.path.join(ROOT, 'tests', 'test_host_router.py')!r}]))\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=580)
    reports = [open(os.path.join(OUT, f)).read()[:3000] for f in os.listdir(OUT)
               if f.startswith("report")]
    tail = res.stdout[-2000:] + res.stderr[-2000:] + "".join(reports)
    assert res.returncode == 0 and not reports, tail
    assert "passed" in res.stdout, tail


def test_plan_cache_eviction_rule_under_sanitizers():
    if not _tool("g++"):
        pytest.skip("needs g++")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "plan_cache_test")
    src = os.path.join(ROOT, "tests", "host_asan", "plan_cache_test.cpp")
    res = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                          "-fno-sanitize-recover=all", "-I" + CSRC, src, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
