"""Builds libmoe_decode.so (gfx950) in place, next to this file.

    python -m fp8_block_scaled_moe_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_decode.so")
SOURCES = ["capi.hip", "route_quant.hip", "expert_gemm.hip", "expert_gemm_wg.hip", "expert_gemm_fp4.hip", "epilogues.hip",
           "boundary.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source flags. The FP4 GEMM feeds every MFMA result straight into FP32
# FMAs; with VGPR-form MFMAs its results need no copies out of the
# accumulation registers (16 instructions per 256-value item otherwise).
# The other kernels keep the default form, which they were measured with.
SOURCE_FLAGS = {"expert_gemm_fp4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know the feature
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    """Compiles every source (in parallel, each with its own flags) and links
    libmoe_decode.so; returns its path."""
    import concurrent.futures
    import tempfile

    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", "-o", obj, os.path.join(CSRC, src)]
            return obj, *_run(cmd, verbose)

        workers = min(len(SOURCES), os.cpu_count() or 1, 8)
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            results = list(pool.map(compile_one, SOURCES))
        for (obj, rc, msgs), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{msgs}")
            if verbose and msgs.strip():
                print(msgs)
        tmp = LIB + f".tmp{os.getpid()}"
        rc, msgs = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                         *[r[0] for r in results]], verbose)
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
