"""Build libsparse_attn.so (HIP for gfx950) in-tree.

Usage: python -m sparse_attention_long_kv_amd.build_lib [--jobs N]

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instruction selection switched off and floating-point contraction disabled
(the kernels spell out each fused multiply-add they want, so fused and
unfused paths round identically).  The host-only planning code is plain C++.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")

HIP_SOURCES = ["api.hip", "append.hip", "indexer.hip", "decode.hip", "linear_gate.hip",
               "noalloc.hip"]
CXX_SOURCES = ["host_plan.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r


def build(jobs=None, verbose=False, out=None, defines=()):
    """Compile and link; `out` overrides the library path, `defines` adds -D flags."""
    tag = "_".join(d.replace("=", "-") for d in defines)
    build_dir = BUILD if not defines else os.path.join(BUILD, "variant_" + tag)
    os.makedirs(build_dir, exist_ok=True)
    extra = ["-D" + d for d in defines]
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmds.append([HIPCC] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(build_dir, src.replace(".cpp", ".o"))
        cmds.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, fut in [(c, ex.submit(_run, c)) for c in cmds]:
            fut.result()
            if verbose:
                print(" ".join(cmd))
    lib = out or LIB
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--out", default=None, help="write the library here instead")
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="extra preprocessor definition for the HIP sources")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.out, tuple(a.defines)))


if __name__ == "__main__":
    main()
