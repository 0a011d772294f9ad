"""Build libcsa.so (gfx950 HIP kernels + the C ABI) in-tree with hipcc.

Usage: python -m long_context_compressed_amd.build [-v]
The kernels are compiled for gfx950 only.  Packed-fp32 instructions are disabled
(-target-feature -packed-fp32-ops) for every device compilation.  The C ABI translation
unit (host validation + dispatch) is plain C++ built with g++.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
# peak-rate probes used only by the benchmark's measured roofline denominators
PROBE_SRC = os.path.join(PKG, "probe", "peaks.hip")
PROBE_LIB = os.path.join(PKG, "libcsa_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=fast",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
             "-I" + os.path.join(ROCM, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    if verbose and r.stdout.strip():
        print(r.stdout)
    return r.stdout


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose=False, jobs=None):
    """Compile every kernel and the ABI, link libcsa.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    jobs = jobs or min(8, max(1, len(hip) + len(cpp)))
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        objs.append(o)
        cmds.append([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        objs.append(o)
        cmds.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, f), "-o", o])
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC] + HIP_FLAGS + ["-shared", PROBE_SRC, "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
