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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the argument
# validation in attn_api.hip (device code is built as usual).  A process that
# loads such a build needs clang's ASan runtime preloaded (asan_runtime()).
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all",
                       "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of the ROCm clang ASan runtime matching HOST_SANITIZE_FLAGS, or None."""
    out = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = out.stdout.strip().splitlines()[-1] if out.returncode == 0 and out.stdout.strip() else ""
    if os.path.isabs(path) and os.path.exists(path):
        return path
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build(verbose: bool = False, extra_flags=(), host_sanitize: bool = False, out: str = None,
          jobs: int = 1) -> str:
    """Compile every source and link libattn.so (or `out`).  `host_sanitize`
    builds the host code with HOST_SANITIZE_FLAGS into a separate object dir."""
    lib = out or LIB
    objdir = os.path.join(ROOT, "_build", "host_sanitize" if host_sanitize else "")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *extra_flags,
               *(HOST_SANITIZE_FLAGS if host_sanitize else []), "-c", "-o", obj, src]
        cmd.remove("-shared")
        cmds.append(cmd)
        objs.append(obj)
    for i in range(0, len(cmds), max(1, jobs)):
        procs = []
        for cmd in cmds[i:i + max(1, jobs)]:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd))
        if any(p.wait() != 0 for p in procs):
            raise subprocess.CalledProcessError(1, "hipcc")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs]
    if host_sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address,undefined", "-shared-libsan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
