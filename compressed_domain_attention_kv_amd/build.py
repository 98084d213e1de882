"""Build libtq.so in-tree for gfx950 with hipcc.

    python compressed_domain_attention_kv_amd/build.py [--jobs N]

Run it as a file: importing the package loads the library it rebuilds.

Every HIP source is compiled with packed-FP32 instructions disabled; the host
core is plain C++17.  The library lands next to this file as ``libtq.so``.
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
OUT = os.path.join(PKG, "libtq.so")
BUILD = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast", "-munsafe-fp-atomics"]

HIP_SOURCES = ["tq_write.hip", "tq_decode.hip", "tq_combine.hip"]
CPP_SOURCES = ["tq_host.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"compile failed: {cmd[-1]}")
    return r


def build(jobs=4, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([HIPCC, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *COMMON, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for r, cmd in zip(ex.map(_run, cmds), cmds):
            if verbose:
                print(" ".join(cmd))
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    shutil.move(tmp, OUT)
    return OUT


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
