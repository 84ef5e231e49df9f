"""Build the gfx950 HIP library ``libqlora_nf4.so`` in-tree.

Every source is compiled with hipcc for gfx950 only, with
``-ffp-contract=off`` (the quantise / dequantise arithmetic must be single
correctly rounded operations; fused multiply-adds are written explicitly where
wanted) and with packed-fp32 instruction selection disabled.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_DIR = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqlora_nf4.so")
SOURCES = ["tables.cpp", "api.cpp", "quant.hip", "gemm.hip", "lora.hip", "gemv.hip", "adamw.hip",
           "merge.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Wall", "-Wno-unused-function"]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source device flags: the decode kernel keeps its MFMA results in VGPRs
# (with AGPR results it holds 16 blocks' results live and fits one wave fewer
# per SIMD); the GEMMs pin their accumulators in AGPRs themselves
EXTRA = {"gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    path = os.path.join(SRC_DIR, src)
    obj = os.path.join(OBJ_DIR, src + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + EXTRA.get(src, []) + ["-x", "hip"]
    cmd += ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
