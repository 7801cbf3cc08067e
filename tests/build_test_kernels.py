"""Build the test-only HIP kernels next to their sources (gfx950), with the
library's own code-generation flags.

    python -m tests.build_test_kernels
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNELS = {"fp8_cvt_sweep.hip": "libkvc_test_fp8_sweep.so", "norm_sweep.hip": "libkvc_test_norm_sweep.so"}
# the library's device helpers (kvc_arch.h) for the kernels that test them
INCLUDES = ["-I", os.path.join(os.path.dirname(HERE), "kv_cache_page_kvc_amd", "csrc")]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def lib_path(source: str) -> str:
    return os.path.join(HERE, KERNELS[source])


def build(verbose: bool = False) -> None:
    for src, so in KERNELS.items():
        tmp = os.path.join(HERE, so + ".tmp")
        cmd = [HIPCC, *FLAGS, *INCLUDES, "-o", tmp, os.path.join(HERE, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed building {so}")
        os.replace(tmp, os.path.join(HERE, so))


if __name__ == "__main__":
    build(verbose=True)
