"""Build libw4a8.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Compiles every ``csrc/*.hip`` into one shared library next to this file.  Flags:
  -O3 --offload-arch=gfx950      CDNA4 only
  -ffp-contract=off              no fused multiply-add unless written explicitly
                                 (the requant's error sums must be exact fp32 ops)
  no -ffast-math, no denormal flushing (fp32 denormals are needed for exact
                                 e2m1 and e8m0 arithmetic)
  -mno-packed-fp32-ops via -target-feature: packed fp32 VALU ops are not emitted
Run as ``python -m w4a8_gemm_amd.build`` or through ``__graft_entry__.build()``.
"""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw4a8.so")
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="w4a8_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            return obj
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, srcs))
        out = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out, LIB)
    return LIB


def asm(src_name: str, out_path: str) -> None:
    """Write the gfx950 assembly of one source (for reading register use and
    instruction selection of our own kernels)."""
    src = os.path.join(CSRC, src_name)
    cmd = [HIPCC, *COMMON, "--cuda-device-only", "-S", src, "-o", out_path]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
