"""Build the gfx950 shared library libqmoe.so in-tree with hipcc.

    python -m quantized_moe_prefill_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
generation disabled, and linked into quantized_moe_prefill_amd/lib/libqmoe.so.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
BUILDDIR = os.path.join(ROOT, "_build")
LIBNAME = "libqmoe.so"
SOURCES = ["api.cpp", "route.hip", "permute.hip", "ffn.hip", "ffn_stream.hip", "small.hip", "ffn_i8.hip",
           "elementwise.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-fPIC",
        "-std=c++17",
        "-Wall",
        "-Wno-unused-function",
        # no packed fp32 (v_pk_*_f32) instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{os.path.join(ROOT, 'include')}",
        f"-I{CSRC}",
    ]


def _compile(src: str) -> str:
    os.makedirs(BUILDDIR, exist_ok=True)
    obj = os.path.join(BUILDDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + common_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if l.strip() and noise not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    """Compile all sources and link the shared library; returns its path."""
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    os.makedirs(LIBDIR, exist_ok=True)
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    # --no-undefined: a kernel whose host-side stub was not emitted must fail
    # the build, not the first launch
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    build(a.jobs)


if __name__ == "__main__":
    main()
