"""Build libgdn.so (HIP kernels + C ABI) and libgdn_peak.so (measured-peak
loops for the benchmark's context figures) for gfx950 with hipcc, in-tree.

Usage: ``python -m linear_attention_sequence_gated_amd.build``.  Objects go to
``_build/`` at the repository root; the shared libraries are written next to
this file so the Python binding finds them.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
PEAK_LIB = os.path.join(PKG, "libgdn_peak.so")
PEAK_SOURCES = ["peak.hip"]
SOURCES = ["chunk_fwd.hip", "chunk_pipe.hip", "chunk_two.hip", "chunk_cx.hip", "chunk_bwd.hip", "tok_bwd.hip", "chunk_grad.hip", "channel_decay.hip", "channel_chunk.hip", "decode.hip", "noalloc.hip", "prologue.hip", "gdn_api.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for device code (the host pass warns that it
# does not know the feature; that warning is expected).
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


# Per-source flags.  channel_chunk.hip rescales its matrix-core accumulators with
# vector instructions every step; the VGPR form of the MFMA instructions keeps
# them in VGPRs instead of copying them to and from AGPRs each time.
# peak.hip needs the same form for its loop of chained accumulations, or the
# register allocator shuffles the accumulators through AGPR copies every round.
EXTRA = {"channel_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {os.path.basename(lib)}:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    allsrc = SOURCES + PEAK_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(allsrc), 8)) as ex:
        objs = dict(zip(allsrc, ex.map(_compile, allsrc)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAK_SOURCES], PEAK_LIB)
    if verbose:
        print(f"built {LIB} and {PEAK_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
