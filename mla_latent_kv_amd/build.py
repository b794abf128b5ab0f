"""Build libmla_decode.so (the HIP kernels and the C ABI) for gfx950 in-tree,
and beside it libmla_decode_debug.so: the same objects except the C ABI,
compiled with MLA_DEBUG_CHECKS (host-side precondition checks before every
launch).

Usage: python -m mla_latent_kv_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla_decode.so")
DEBUG_LIB = os.path.join(HERE, "libmla_decode_debug.so")
SOURCES = ["api.hip", "check.cpp", "prep.hip", "prep_wide.hip", "attn.hip", "merge.hip", "wpack.hip", "append.hip", "oproj.hip", "qproj.hip", "naive.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-FP32 VALU forms stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the MLA decode library needs ROCm's hipcc")
    return path


def _compile(src: str, debug: bool = False) -> str:
    stem = os.path.splitext(src)[0] + ("_debug" if debug else "")
    out = os.path.join(OBJ, stem + ".o")
    defs = ["-DMLA_DEBUG_CHECKS"] if debug else []
    cmd = [hipcc(), *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return out


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link the release and debug libraries; returns
    the release library's path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [("api.hip", True)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    release = objs[:len(SOURCES)]
    _link(release, LIB)
    _link([objs[-1]] + release[1:], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
