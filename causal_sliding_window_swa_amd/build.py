"""Builds libswa.so in-tree with hipcc for gfx950.

    python -m causal_sliding_window_swa_amd.build

Every .hip/.cpp file under csrc/ is compiled to an object (in parallel, under
_build/) and linked into causal_sliding_window_swa_amd/libswa.so; the
measurement probe under measure/ goes into libswa_measure.so (bench.py only).  HIP code is
compiled with packed fp32 arithmetic disabled (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libswa.so")
# measurement support for bench.py (a streaming-read probe), not the library
MEASURE = os.path.join(PKG, "measure")
MEASURE_OUT = os.path.join(PKG, "libswa_measure.so")
BUILD_DIR = os.path.join(PKG, "_build")
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + CFLAGS + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    msrcs = [os.path.join(MEASURE, f) for f in sorted(os.listdir(MEASURE)) if f.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(msrcs))) as ex:
        objs = list(ex.map(_compile, srcs + msrcs))
    _link(objs[:len(srcs)], OUT)
    _link(objs[len(srcs):], MEASURE_OUT)
    if verbose:
        print("built", OUT, "and", MEASURE_OUT)
    return OUT


if __name__ == "__main__":
    build()
