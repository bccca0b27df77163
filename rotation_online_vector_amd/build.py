"""Build libtq.so (HIP for gfx950) in-tree with hipcc.

    python -m rotation_online_vector_amd.build

Every HIP source is compiled with packed fp32 instructions disabled
(-target-feature -packed-fp32-ops); the host compiler pass warns that it does
not know the feature, which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libtq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kernels.hip", "encode128.hip", "score128.hip", "score_f16.hip", "tq_api.cpp",
           "host_tables.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "not a recognized feature for this target"
    out = "\n".join(l for l in p.stdout.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    if out.strip():
        print(out)


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(LIBDIR, src.replace(".", "_") + ".o")
    cmd = [HIPCC, "--offload-arch=" + ARCH] + COMMON + ["-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print("[build]", src, flush=True)
    _run(cmd)
    return obj


def build(verbose=True):
    """Compile every source (in parallel) and link libtq.so."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda src: _compile(src, verbose), SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
