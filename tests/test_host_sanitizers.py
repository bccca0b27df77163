"""The library's host code (plan tables, Lloyd-Max solver, Philox generators, argument
checks: `tq_api.cpp`, `host_tables.cpp`) built with the host compiler under the address and
undefined-behaviour sanitizers, with leak detection, and driven by the two plain-C programs
in tests/c: the C ABI checks and a sweep of plan shapes.  The kernels are not part of this
build: tests/c/host_stubs.cpp stands in for the launchers and for the HIP calls the host code
makes (host memory as device memory), so plan creation runs to the end on any machine."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rotation_online_vector_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _tools():
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    hip_inc = "/opt/rocm/include"
    if gxx is None or gcc is None or not os.path.isdir(os.path.join(hip_inc, "hip")):
        pytest.skip("g++/gcc or the HIP headers are not available")
    return gxx, gcc, hip_inc


@pytest.fixture(scope="module")
def host_objects(tmp_path_factory):
    gxx, gcc, hip_inc = _tools()
    out = tmp_path_factory.mktemp("san")
    objs = []
    for src in (os.path.join(CSRC, "tq_api.cpp"), os.path.join(CSRC, "host_tables.cpp"),
                os.path.join(ROOT, "tests", "c", "host_stubs.cpp")):
        o = str(out / (os.path.basename(src) + ".o"))
        subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", hip_inc]
                       + SAN + ["-c", src, "-o", o], check=True, capture_output=True, text=True)
        objs.append(o)
    return gxx, gcc, out, objs


@pytest.mark.parametrize("program", ["c_abi_host.c", "host_sweep.c"])
def test_host_code_clean_under_sanitizers(host_objects, program):
    gxx, gcc, out, objs = host_objects
    src = os.path.join(ROOT, "tests", "c", program)
    o = str(out / (program + ".o"))
    exe = str(out / program.replace(".c", ""))
    subprocess.run([gcc, "-std=c99", "-O1", "-g", "-Wall", "-Werror", "-I",
                    os.path.join(ROOT, "include")] + SAN + ["-c", src, "-o", o],
                   check=True, capture_output=True, text=True)
    subprocess.run([gxx] + SAN + [o] + objs + ["-o", exe, "-lm"], check=True,
                   capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.strip().endswith("all passed")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
