"""Build libtka.so (gfx950) in-tree with hipcc.

Usage: python top_sparse_attention_topk_amd/build.py   (run as a file: it must not
import the package, whose binding loads the library being built)
Each .hip source is compiled to an object in _build/ (in parallel), then
linked into top_sparse_attention_topk_amd/libtka.so; the benchmark's
streaming-read probe (csrc/probe/) into libtka_probe.so beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libtka.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "score.hip", "select.hip", "gather.hip", "cache.hip", "hisa.hip"]
PROBE_SOURCES = ["probe/stream_read.hip"]
PROBE_OUT = os.path.join(PKG, "libtka_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(7, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], OUT)
    # the benchmark's streaming-read probe, a library of its own (not part of libtka)
    _link(objs[len(SOURCES):], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build()
