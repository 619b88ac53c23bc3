"""Builds the gfx950 shared library libttt.so in-tree with hipcc.

Usage: python -m linear_attention_chunk_amd.build_lib   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libttt.so")
SOURCES = ["errors.hip", "profile.hip", "ttt_layer.hip", "ttt_backward.hip", "ttt_full_bwd.hip", "linattn.hip",
           "swa.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Extra flags per source.  The sliding-window kernel applies the softmax and its rescale to the
# accumulators of its second product, so they belong in VGPRs: with the compiler's default placement
# in AGPRs every key block moved hundreds of values between the two register files.
EXTRA_FLAGS = {"swa.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    return r.returncode, err


def build(verbose: bool = False) -> str:
    """Compiles every HIP source (in parallel, each to an object) and links libttt.so (always
    rebuilds); returns the library path."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_obj")
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append((obj, [hipcc(), *flags, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, cmd), (rc, err) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {os.path.basename(obj)}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([hipcc(), *HIPCC_FLAGS, *[o for o, _ in jobs], "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
