"""Builds libattn_hd512.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled for gfx950 only, with packed fp32 VALU
ops disabled (-packed-fp32-ops), then linked into one shared library beside
this file.  A second library, libattn_hd512_delay.so, is the same sources
built with -DATTN_RACE_DELAY: wave-dependent sleeps after every LDS refill
load and before every workgroup barrier, for the tests that look for races
(it must reproduce the normal build's results bit for bit).  Run
`python -m attention_hd512_gqa_amd.build` or call build().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_hd512.so")
LIB_DELAY = os.path.join(HERE, "libattn_hd512_delay.so")
OBJDIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, objdir: str, extra) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles both libraries (normal and delay-injected); returns the normal one's path."""
    srcs = sources()
    variants = [(LIB, OBJDIR, []), (LIB_DELAY, OBJDIR + "_delay", ["-DATTN_RACE_DELAY"])]
    jobs = []
    for _, objdir, extra in variants:
        os.makedirs(objdir, exist_ok=True)
        jobs += [(src, objdir, extra) for src in srcs]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    for k, (lib, _, _) in enumerate(variants):
        _link(objs[k * len(srcs):(k + 1) * len(srcs)], lib)
    if verbose:
        print(f"built {LIB} and {os.path.basename(LIB_DELAY)} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
