"""Builds librtlynx.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into activation_sparse_gemm_token_amd/librtlynx.so.  Always
rebuilds.  Run as ``python -m activation_sparse_gemm_token_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librtlynx.so")
# The matrix-instruction rate measurement (bench.py --mfma-rates): not part
# of librtlynx, built beside it.
MB_SRC = os.path.join(PKG, "microbench", "mfma_rates.hip")
MB_LIB = os.path.join(PKG, "libmfma_rates.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    # no packed-FP32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags.  sparse_gemm: MFMA accumulators and operands in
# the VGPR form -- with the default heuristic its 256-register accumulator
# tile splits between VGPRs and AGPRs and values spill to scratch, whose
# reloads (vector-memory operations) would drain the DMA pipeline.  (The
# dense kernel is faster in the default form.)
EXTRA = {
    "sparse_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), "-x", "hip", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{res.stderr}")
    if err:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    mb_obj = _compile(MB_SRC)
    tmp = MB_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, mb_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, MB_LIB)
    if verbose:
        print(f"built {LIB} and {MB_LIB}")
    return LIB


if __name__ == "__main__":
    build()
