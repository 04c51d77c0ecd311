"""Build libqmm.so (the HIP kernels and the C ABI of include/qmm.h) for gfx950.

Compiles every source in csrc/ with hipcc into one shared library next to this
file.  Run as ``python -m gguf_block_quant_qmm_amd.build`` or through
``__graft_entry__.build()``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqmm.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-f32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(p, verbose):
    _, err = p.communicate()
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (err or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed ({p.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, out: str | None = None, defines: list[str] | None = None) -> str:
    """Compile every source (in parallel, one object each) and link libqmm.so.

    out: another path for the library; defines: extra -D flags (e.g. QMM_TUNING
    for a measurement build that reads its tuning levers from the environment).
    """
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib = out or LIB
    objdir = os.path.join(ROOT, "_build", os.path.basename(lib) + ".obj")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    dflags = [f"-D{d}" for d in (defines or [])]
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append(_run([hipcc, *HIPCC_FLAGS, *dflags, *inc, "-c", src, "-o", obj], verbose))
    for p in procs:
        _finish(p, verbose)
    tmp = lib + ".tmp"
    _finish(_run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose), verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
