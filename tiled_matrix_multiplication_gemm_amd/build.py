"""Build step of libmi355gemm.so for gfx950, in-tree: the host code and each
table row compile as separate translation units, in parallel, then link into
one shared library.

Usage: python -m tiled_matrix_multiplication_gemm_amd.build [--resource-usage]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB_NAME = "libmi355gemm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)


def sources():
    return [os.path.join(CSRC, "mg_api.hip"), os.path.join(CSRC, "mg_f32.hip")] + sorted(
        glob.glob(os.path.join(CSRC, "mg_row*.hip")))


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _run(cmd):
    return subprocess.run(cmd, capture_output=True, text=True)


def build(resource_usage: bool = False, verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(p).replace(".hip", ".o")) for p in srcs]
    cmds = []
    for src, obj in zip(srcs, objs):
        cmd = [HIPCC, *FLAGS, "-c"]
        if resource_usage:
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        cmds.append(cmd + ["-o", obj, src])
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        procs = list(ex.map(_run, cmds))
    for c, p in zip(cmds, procs):
        if p.returncode != 0:
            sys.stderr.write(p.stderr)
            raise RuntimeError("hipcc failed (exit %d): %s" % (p.returncode, c[-1]))
    if resource_usage:
        with open(os.path.join(CSRC, "_resource_usage.txt"), "w") as f:
            for p in procs:
                f.write(p.stderr)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    p = _run(link)
    if p.returncode != 0:
        sys.stderr.write(p.stderr)
        raise RuntimeError("link failed (exit %d)" % p.returncode)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
    print(LIB_PATH)
