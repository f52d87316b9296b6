"""Build libfa2.so (HIP, gfx950) in-tree with hipcc.

    python -m exact_attention_fa2_amd.build            # compile everything
    python -m exact_attention_fa2_amd.build --asm DIR  # also keep gfx950 assembly

Packed-FP32 instructions are switched off for all device code; only the
symbols of include/fa2.h are exported.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa2.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "fwd_f32.hip", "fwd_mfma.hip", "decode.hip", "bwd.hip", "bwd_f32.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        if asm_dir and src.endswith(".hip"):
            os.makedirs(asm_dir, exist_ok=True)
            cmd += ["--save-temps"]
        r = subprocess.run(cmd, cwd=asm_dir or BUILD_DIR, capture_output=True, text=True)
        msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in x and x.strip())
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
        if verbose and msg:
            print(msg, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH, "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep gfx950 assembly in this directory")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.asm, args.v))


if __name__ == "__main__":
    main()
