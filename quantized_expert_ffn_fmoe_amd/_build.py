"""Compile libfmoe.so (the HIP library) for gfx950, in-tree.

Every .hip source under csrc/ is compiled to an object in parallel, then linked into a
shared library next to this file. Always recompiles (the build check must see every
source compile).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libfmoe.so")

HIPCC = os.environ.get("HIPCC", "hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
         # packed fp32 vector instructions stay off: hipcc -O3 would otherwise form them
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, obj: str, extra=()) -> None:
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(jobs: int = 8, so: str = SO, extra=()) -> str:
    """Compile every source into `so` (default: the library itself; the measurement package
    builds a phase-traced copy elsewhere with extra=["-DFMOE_TRACE"])."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with tempfile.TemporaryDirectory(prefix="fmoe_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s)[:-4] + ".o") for s in srcs]
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda a: _compile(a[0], a[1], extra), zip(srcs, objs)))
        tmp_so = so + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_so] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_so, so)
    return so


if __name__ == "__main__":
    print(build())
