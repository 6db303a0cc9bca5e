"""Build the q8stream shared library (gfx950) in-tree with hipcc.

Each source is compiled to an object in ``_build/`` (in parallel), then linked
into ``int8_weight_streaming_amd/libq8stream.so``; the benchmark's measurement
probes are linked into their own ``libq8probe.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq8stream.so")

SOURCES = ["q8_api.cpp", "q8_quantize.hip", "q8_skinny.hip", "q8_skinny_mfma.hip", "q8_prefill.hip", "q8_attn.hip",
           "q4_skinny.hip", "q8_fused.hip", "q8_prefill_frag.hip"]
PROBE_SOURCES = ["q8_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libq8probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I", INCLUDE, "-I", CSRC]
# Packed fp32 VALU instructions are kept off for all device code.  Matrix-core
# results are written to ordinary VGPRs (no copies out of accumulation
# registers before the fp32 fold).  Kernel arguments (up to 16 dwords) are
# preloaded into SGPRs at wave launch, so a kernel does not start by waiting
# for its argument loads (code built this way keeps a fallback entry that
# loads them, for firmware without preloading); worth 0.26 us per launch in a
# graph of 513 decode products.
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=true",
          "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
