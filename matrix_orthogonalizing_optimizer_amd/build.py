"""Build libmuon.so (HIP, gfx950) in-tree with hipcc.

``python -m matrix_orthogonalizing_optimizer_amd.build`` compiles every
source under ``csrc/`` for gfx950 and links the shared library next to this
file.  Objects go to ``_build/`` at the repository root.
"""

from __future__ import annotations

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
LIB = os.path.join(PKG, "libmuon.so")
SOURCES = ["ns_gemm.hip", "ns_small.hip", "elementwise.hip", "svd_entropy.hip", "muon_api.hip",
           "svd_api.hip", "muon_noalloc.hip"]
# roofline probes of the benchmark: a library of their own, not the optimizer's ABI
PROBE_LIB = os.path.join(PKG, "libmoprobe.so")
PROBE_SOURCES = ["peak_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep private arrays out of LDS: LDS holds only the staged tiles
    "-mllvm", "-disable-promote-alloca-to-lds=true",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # host-pass notice
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _link(objs, lib):
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    # every symbol must resolve (a kernel whose host-side stub was not
    # emitted would otherwise only fail when the library is first loaded)
    _run(["python3", "-c", f"import ctypes; ctypes.CDLL({tmp!r}, mode=ctypes.RTLD_LOCAL)"])
    shutil.move(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile all sources, link ``libmuon.so`` and the probe library;
    returns the path of ``libmuon.so``."""
    os.makedirs(BUILD, exist_ok=True)
    cmds = []

    def objs_of(srcs):
        out = []
        for src in srcs:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            out.append(obj)
            cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return out

    objs = objs_of(SOURCES)
    probe_objs = objs_of(PROBE_SOURCES)
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    _link(objs, LIB)
    _link(probe_objs, PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
