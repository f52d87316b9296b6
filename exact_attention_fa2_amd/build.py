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
# Measurement builds beside the product library: (file name, source rebuilt
# with extra flags, flags); the other objects are shared with libfa2.so.
VARIANTS = [
    # 2 of every 8 exponential pairs of the f16/bf16 forward on the FMA path
    # (polynomial exp2), to time that lever in the kernel and check its parity
    ("libfa2_polyexp.so", "fwd_mfma.hip", ["-DFA2_POLY_EXP=2"]),
]
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

    def compile_one(src, tag="", extra=()):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + tag + ".o")
        cmd = [hipcc, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + list(extra)
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

    jobs = [(src, "", ()) for src in SOURCES]
    jobs += [(src, "." + name, tuple(flags)) for name, src, flags in VARIANTS]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: compile_one(*j), jobs))
    base = objs[:len(SOURCES)]

    def link(out, objects):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc, "-shared", "-o", tmp] + objects + ["--offload-arch=" + ARCH, "-fPIC"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, out)

    link(OUT, base)
    for (name, src, _), obj in zip(VARIANTS, objs[len(SOURCES):]):
        link(os.path.join(PKG, name), [obj if s == src else o for s, o in zip(SOURCES, base)])
    return OUT


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep gfx950 assembly in this directory")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.asm, args.v))


if __name__ == "__main__":
    main()
