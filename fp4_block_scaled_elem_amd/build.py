"""Build libmq.so (HIP for gfx950) in place, with hipcc.

    python -m fp4_block_scaled_elem_amd.build [-v]

Every source is compiled for gfx950 only, with IEEE-exact float semantics
(-ffp-contract=off, correctly rounded division, no fast-math) so that the
quantizer is bit-reproducible, and with packed-fp32 instructions disabled.
Objects go to fp4_block_scaled_elem_amd/_build/, the library next to this
file.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmq.so")
SOURCES = ("api.hip", "quant.hip", "gemm.hip", "gemv.hip", "gemv_nvfp4.hip", "producer.hip", "codec_check.hip", "peak.hip")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def obj(src):
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([cc, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", o], verbose)
        return o

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(obj, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
