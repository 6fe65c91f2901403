"""Build libq8kv.so (the HIP kernels and their C ABI) for gfx950, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "q8kv.hip")
LIB = os.path.join(HERE, "libq8kv.so")
EXAMPLE_SRC = os.path.join(HERE, "csrc", "q8kv_example.c")
EXAMPLE = os.path.join(HERE, "q8kv_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every atomic here is issued by one thread: the atomic optimizer's
    # cross-lane reduction only adds a wait for each atomic's result before
    # the next one can go out
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    # leading scalar kernel arguments arrive preloaded in SGPRs (the decode
    # kernel's first dependent loads then need no argument-block round trip)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    """Compile csrc/q8kv.hip into libq8kv.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def example_command(out=EXAMPLE):
    """The host compiler line of the plain C caller (csrc/q8kv_example.c),
    linked against libq8kv.so (found next to the binary at run time) and the
    HIP runtime."""
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), EXAMPLE_SRC,
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", HERE, "-lq8kv",
            "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-Wl,-rpath,$ORIGIN", "-o", out]


def build_example(verbose=False):
    """Compile the C example against the built library (always recompiles)."""
    tmp = EXAMPLE + ".tmp"
    cmd = example_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, EXAMPLE)
    return EXAMPLE


if __name__ == "__main__":
    build(verbose=True)
    build_example(verbose=True)
