"""Build libmla.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libmla.so")
PROBE_PATH = os.path.join(PKG, "libmlaprobe.so")       # measurement probe (profiles only)
PROBE_SOURCES = [os.path.join(PKG, "csrc", "mla_probe.hip")]
SOURCES = [os.path.join(PKG, "csrc", "libmla.hip"), os.path.join(PKG, "csrc", "mla_proj.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc(sources, path, verbose):
    tmp = path + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *sources, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, path)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the HIP sources into libmla.so (and the measurement probe into
    libmlaprobe.so) next to this file."""
    if not force and os.path.exists(LIB_PATH) and os.path.exists(PROBE_PATH):
        return LIB_PATH
    _hipcc(SOURCES, LIB_PATH, verbose)
    _hipcc(PROBE_SOURCES, PROBE_PATH, verbose)
    return LIB_PATH
