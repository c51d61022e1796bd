"""Build step for libattn.so: every HIP source under csrc/ compiled for gfx950.

Flags: -O3, C++17, hidden visibility (only the extern "C" entry points of
include/attn.h are exported) and packed-fp32 instruction selection disabled.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Extra flags per source.  The prefill kernel never produces or consumes a
# NaN on valid inputs, so it is built without IEEE NaN quieting: fmaxf then
# lowers to v_max3_f32 without canonicalising every MFMA result first.
PER_FILE_FLAGS = {
    "prefill_fwd.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
    # MFMA results in VGPRs: the score accumulators feed the softmax VALU
    # directly (the Q fragments, pure MFMA operands, are pinned to AGPRs)
    "prefill_dual.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *extra_flags,
               "-c", "-o", obj, src]
        cmd.remove("-shared")
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
