"""Compile the HIP library (gfx950) into ``libchp.so`` next to this file."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libchp.so")
OBJDIR = os.path.join(ROOT, "_build", "chp")
SOURCES = ["api.hip", "k_scan.hip", "k_build.hip", "k_rate.hip", "k_contract.hip", "k_coarse.hip",
           "k_bitmap.hip", "k_eval.hip", "k_rate_inc.hip", "k_rate_incq.hip",
           "k_sort.hip", "k_leftover.hip", "k_gain.hip", "k_match_dp.hip",
           "k_refine.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE,
         # packed-fp32 instructions stay off (they are not needed here)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# The rating kernel takes work items from a counter ahead of use; the
# compiler's wave-level atomic rewrite would wait for each result at once.
EXTRA = {"k_rate.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source (always) and link libchp.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
