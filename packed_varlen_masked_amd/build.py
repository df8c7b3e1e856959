"""Builds libflashmask_mi355.so in-tree with hipcc for gfx950.

Every HIP source is compiled for gfx950 only; packed fp32 VALU ops are
switched off for device code.  The library lands next to this file, where
the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libflashmask_mi355.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["fm_api.cpp", "fm_plan.hip", "fm_attn_bf16.hip", "fm_attn_f32.hip", "fm_bwd_bf16.hip", "fm_rope.hip"]
ARCH = "gfx950"
# Per-source compiler flags beyond compile_flags() (none at present).
EXTRA_FLAGS = {}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=%s" % ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # every atomic in these kernels is issued by a single lane; the
            # atomic optimizer would make its result needed at once
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
            "-Wno-unused-variable"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source (always, also when a library exists) and link."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc] + compile_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        objs.append(obj)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if verbose or p.returncode:
            sys.stderr.write("\n".join(lines) + ("\n" if lines else ""))
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: %s" % ", ".join(failed))
    tmp = LIB_PATH + ".tmp"
    link = [cc, "-shared", "-fPIC", "--offload-arch=%s" % ARCH, "-o", tmp] + objs
    out = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if out.returncode:
        sys.stderr.write(out.stdout.decode(errors="replace"))
        raise RuntimeError("link failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
