"""Build libsfa.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python fixed_offset_gather_amd/build.py  (or __graft_entry__.build()); a plain script, so
it runs before the package (which needs the library) can be imported.
Objects go to _build/ at the repository root; the shared library is written
next to this file so that the Python binding (and a copy of the tree sent to
a GPU machine) finds it without installation.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsfa.so")
PROBE = os.path.join(PKG, "lds_probe")

ARCH = "gfx950"
HIP_SOURCES = ["sfa_api.hip", "sfa_fwd.hip", "sfa_bwd.hip", "sfa_noalloc.hip"]
CXX_SOURCES = ["sfa_producers.cpp"]

# Packed FP32 instructions are disabled for all device code.  The tied
# two-operand v_dot2c_f32_f16 and v_dot2c_f32_bf16 are disabled too: a dot
# that starts from zero then needs a v_mov per accumulator, while the
# three-operand v_dot2_f32_f16 and v_dot2_f32_bf16 (same issue rate) take
# the 0 as an inline constant.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xclang", "-target-feature", "-Xclang", "-dot5-insts",
    "-Xclang", "-target-feature", "-Xclang", "-dot13-insts",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsfa)")


def build(verbose=False):
    """Compile every source and link libsfa.so.  Raises on failure."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc, "-c", os.path.join(CSRC, src), "-o", obj] + HIP_FLAGS + inc
        jobs.append((src, cmd))
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        cmd = ["g++", "-c", os.path.join(CSRC, src), "-o", obj, "-O2", "-std=c++17",
               "-fPIC", "-Wall"] + inc
        jobs.append((src, cmd))
        objs.append(obj)
    procs = []
    for src, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join("== %s ==\n%s" % f for f in failed)
        raise RuntimeError("libsfa build failed:\n" + msg)
    tmp = LIB + ".tmp"
    link = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("libsfa link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    # the LDS access-pattern calibration program used with the bank-conflict
    # counters (not part of the library)
    probe = [hipcc, os.path.join(CSRC, "lds_probe.hip"), "-o", PROBE] + [f for f in HIP_FLAGS if f != "-fPIC"]
    if verbose:
        print(" ".join(probe), flush=True)
    r = subprocess.run(probe, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("lds_probe build failed:\n" + r.stdout.decode(errors="replace"))
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
