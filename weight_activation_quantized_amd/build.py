"""Builds libmixllm.so (HIP kernels for gfx950 + host packer) in-tree.

    python -m weight_activation_quantized_amd.build [--variants]

``--variants`` also builds the measured alternatives of the tile GEMM (same C ABI, one
compile-time switch each) as libmixllm_<name>.so next to the library:

    fold_bias  the float-bits int-to-float conversion: the partial's MFMA chain starts from
               the integer 0x4B400000 and one exact float subtraction replaces
               v_cvt_f32_i32
    zero_pre   4-bit zero points subtracted from the codes before the matrix cores with
               byte-wise integer ops, instead of the per-group matrix-core correction

Every source is compiled with hipcc for --offload-arch=gfx950 with packed-FP32
instructions disabled and floating-point contraction off (the kernels write their
fused multiply-adds explicitly), then linked into ``libmixllm.so`` next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmixllm.so")

VARIANTS = {"fold_bias": ("MIXLLM_FOLD_BIAS=1",), "zero_pre": ("MIXLLM_ZERO_PRE=1",)}

SOURCES = ["mixllm_pack.cpp", "mixllm_assign.cpp", "mixllm_quant_act.hip", "mixllm_gemm.hip"]
ARCH = os.environ.get("MIXLLM_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmixllm.so)")


COMMON = ["-std=c++17", "-O3", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compiles every source and links ``out``; ``defines`` are extra -D flags (tuning
    knobs such as ring depths)."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        tag = ("_" + "_".join(d.replace("=", "") for d in defines)) if defines else ""
        obj = os.path.join(BUILD, src + tag + ".o")
        dflags = [f"-D{d}" for d in defines]
        if src.endswith(".hip"):
            cmd = [cc, "-x", "hip", *COMMON, *dflags, *DEVICE, "-c", path, "-o", obj]
        else:
            cmd = [cc, "-x", "c++", *COMMON, *dflags, "-c", path, "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([cc, *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs, "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(tmp, out)
    return out


def variant_path(name: str) -> str:
    return os.path.join(HERE, f"libmixllm_{name}.so")


def build_variants(verbose: bool = False):
    return [build(verbose, variant_path(name), defs) for name, defs in VARIANTS.items()]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--variants" in sys.argv:
        for path in build_variants(verbose="-v" in sys.argv):
            print(path)
