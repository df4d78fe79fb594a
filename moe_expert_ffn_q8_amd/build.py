"""Build libq8moe.so (the HIP kernels + C ABI) in-tree for gfx950.

Every HIP source is compiled with hipcc for gfx950 only, at -O3, without
fast-math (the quantizer relies on IEEE division, roundf and RNE fp16
conversion), and with packed fp32 instructions disabled in the device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libq8moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quantize.hip", "stream.hip", "step.hip", "ffn.hip", "small_m.hip", "moe.hip",
           "moe_gemm.hip", "moe_r8.hip", "gemm.hip", "r8.hip", "r8_mm.hip", "kquant.hip", "probe.hip",
           "abi.cpp"]

# no packed fp32 instructions in device code; MFMA results in VGPRs (the
# rescale of each int32 block tile then needs no accumulator-register copies)
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src, verbose, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE_FLAGS, *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature name: drop that warning
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(verbose=False, lib=LIB, build_dir=BUILD, defines=()):
    """Compile every source and link `lib`.  `defines` are extra -D options
    (build-time tuning knobs such as Q8_WEIGHT_CACHE_POLICY)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
