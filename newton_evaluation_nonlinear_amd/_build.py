"""Compile libpn.so in-tree for gfx950 with hipcc.

    python -m newton_evaluation_nonlinear_amd._build

Each source is compiled to an object in parallel (the device code of every
file is self-contained), then the objects are linked into libpn.so; the
ceiling microbenchmarks (pn_ceiling.hip) become libpn_ceiling.so.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpn.so")
# the ceiling microbenchmarks (a measurement tool, include/pn_ceiling.h)
CEILING_LIB = os.path.join(HERE, "libpn_ceiling.so")
CEILING_SOURCES = ["pn_ceiling.hip"]

SOURCES = ["pn_api.cpp", "pn_diag.hip", "pn_cell.hip", "pn_dense.hip", "pn_scan.hip", "pn_static.hip", "pn_small.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 ALU forms stay off: keep every FP32 op scalar
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libpn.so")
    return r.stderr


def build(verbose=False):
    with tempfile.TemporaryDirectory(prefix="pn_build_") as tmpd:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmpd, src + ".o")
            objs.append(obj)
            cmds.append([hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c",
                                             os.path.join(CSRC, src), "-o", obj])
        cobjs = []
        for src in CEILING_SOURCES:
            obj = os.path.join(tmpd, src + ".o")
            cobjs.append(obj)
            cmds.append([hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c",
                                             os.path.join(CSRC, src), "-o", obj])
        workers = min(len(cmds), max(1, (os.cpu_count() or 1)))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            logs = list(ex.map(_run, cmds))
        tmp = LIB + ".tmp"
        logs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs))
        ctmp = CEILING_LIB + ".tmp"
        logs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", ctmp] + cobjs))
    if verbose:
        for cmd in cmds:
            print(" ".join(cmd), flush=True)
        for lg in logs:
            lines = [ln for ln in lg.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
            if lines:
                sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    os.replace(ctmp, CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
