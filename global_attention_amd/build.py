"""Build libbeam_attn.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m global_attention_amd.build   (or global_attention_amd.build.build())
The library is written next to this file; object files go to _build/.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbeam_attn.so")
SOURCES = ["beam_attn.hip", "prologue.hip", "prefill.hip", "decode.hip", "router.hip", "gemm.hip", "probe.hip",
           "kv_layout.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(7, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_kernel_stubs(lib: str) -> None:
    """Every kernel the host code launches must have its launch stub in the
    library: the compiler's host pass can drop one without an error."""
    try:
        r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    except FileNotFoundError:
        return
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError(f"kernel launch stubs missing from {lib}: {missing}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
