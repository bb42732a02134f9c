"""Build libtpconv.so in-tree for gfx950.

Steps: compile and run the CG code generator (host C++) to emit the device
coupling code, compile every translation unit with hipcc in parallel, link
the shared library next to this file.  Usage: python -m
equivariant_gnn_tensor_receiver_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
GEN = os.path.join(BUILD, "gen")
LIB = os.path.join(HERE, "libtpconv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay disabled: ordinary fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-munsafe-fp-atomics",
]
# (object name, source, extra defines)
STREAM_VARIANTS = [
    ("fwd_f32", "kFwd", 1), ("fwd_bf16", "kFwd", 0),
    ("jvp_f32", "kJvp", 1), ("jvp_bf16", "kJvp", 0),
    ("snd_f32", "kSnd", 1), ("sndt_f32", "kSndT", 1),
]
POS_VARIANTS = [("bpos_f32", "float", 0), ("bpos_bf16", "uint16_t", 0), ("hess_f32", "float", 1),
                ("hess_bf16", "uint16_t", 1)]
# The edge streams keep their matrix-core accumulators in ordinary VGPRs
# (the accumulation registers would otherwise be copied back and forth).
STREAM_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
UNITS = ([(f"stream_{n}", "stream_gf.hip", STREAM_FLAGS + [f"-DTP_MODE={m}", f"-DTP_LO={lo}",
                                                          f"-DTP_LAUNCHER=launch_stream_{n}"])
          for n, m, lo in STREAM_VARIANTS]
         + [(f"stream_{n}", "stream_pos.hip", STREAM_FLAGS + [f"-DTP_FT={t}", f"-DTP_HESS={h}",
                                                             f"-DTP_LAUNCHER=launch_stream_{n}"])
            for n, t, h in POS_VARIANTS]
         + [(u, u + ext, []) for u, ext in (("gemm", ".hip"), ("channelwise", ".hip"), ("graph", ".hip"), ("radial", ".hip"), ("fixed", ".hip"),
                                             ("scratch", ".hip"), ("ragged", ".hip"), ("api", ".cpp"),
                                             ("stream_dispatch", ".cpp"), ("plan", ".cpp"),
                                             ("timing", ".cpp"))])


def run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def generate():
    os.makedirs(GEN, exist_ok=True)
    exe = os.path.join(BUILD, "cg_codegen")
    run(["g++", "-O2", "-std=c++17", os.path.join(CSRC, "cg_codegen.cpp"), os.path.join(CSRC, "plan.cpp"),
         "-I", os.path.join(ROOT, "include"), "-o", exe])
    run([exe, os.path.join(GEN, "cg_tables.inc")])


def _newest_input(src: str) -> float:
    """Newest of a unit's source, every header, the generated tables and this script."""
    files = ([os.path.join(CSRC, src), os.path.join(ROOT, "include", "tpconv.h"), __file__]
             + glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(GEN, "*")))
    return max(os.path.getmtime(f) for f in files if os.path.isfile(f))


def compile_one(unit, incremental=False):
    name, src, defines = unit
    obj = os.path.join(BUILD, name + ".o")
    if incremental and os.path.exists(obj) and os.path.getmtime(obj) > _newest_input(src):
        return obj
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    run([HIPCC] + HIP_FLAGS + defines + ["-I", GEN, "-I", CSRC, "-I", os.path.join(ROOT, "include")] + lang +
        ["-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def build(jobs: int = 8, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every unit (incremental=True skips objects newer than all sources) and link."""
    os.makedirs(BUILD, exist_ok=True)
    tables = os.path.join(GEN, "cg_tables.inc")
    gen_inputs = [os.path.join(CSRC, f) for f in ("cg_codegen.cpp", "plan.cpp", "plan.h")]
    if not (incremental and os.path.exists(tables)
            and os.path.getmtime(tables) > max(os.path.getmtime(f) for f in gen_inputs)):
        generate()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda u: compile_one(u, incremental), UNITS))
    tmp = LIB + ".tmp"
    run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--incremental", action="store_true", help="skip objects newer than every source")
    args = ap.parse_args()
    build(args.jobs, verbose=True, incremental=args.incremental)
    sys.exit(0)
