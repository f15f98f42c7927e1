"""Builds libhsa_attn.so (all HIP sources, gfx950) in-tree next to this file.

    python -m hierarchical_sparse_attention_hsa_amd.build

Compiles every csrc/*.hip with hipcc for gfx950 and links one shared
library, and the same sources with HSA_ATTN_DEBUG=1 into
libhsa_attn_debug.so (poisoned workspaces and index checks); the benchmark's read-bandwidth probe (measure/stream_read.hip) is
built into a library of its own, libhsa_attn_stream.so, and the MFMA/VALU
overlap probe (measure/mfma_valu_overlap.hip) into an executable next to
its source.  No fast-math and no denormal flushing; packed fp32 VALU ops are
disabled for device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhsa_attn.so")
# the same sources with HSA_ATTN_DEBUG=1: poisoned workspaces, index checks
DEBUG_BUILD = os.path.join(HERE, "_build_debug")
DEBUG_LIB = os.path.join(HERE, "libhsa_attn_debug.so")
# the benchmark's read-bandwidth probe, a library of its own (measure/)
STREAM_SRC = os.path.join(HERE, "measure", "stream_read.hip")
STREAM_LIB = os.path.join(HERE, "libhsa_attn_stream.so")
# a standalone probe of MFMA / VALU overlap (measure/; an executable)
OVERLAP_SRC = os.path.join(HERE, "measure", "mfma_valu_overlap.hip")
OVERLAP_EXE = os.path.join(HERE, "measure", "mfma_valu_overlap")
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the scores and outputs feed VALU
    # code directly, without v_accvgpr_read copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # inputs are finite by contract and no kernel produces a NaN, so min/max
    # need no NaN quieting
    "-fno-honor-nans",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    """All HIP sources, minus prefill instantiation units left out by
    HSA_ATTN_PREFILL_VARIANTS (comma list such as "bf16_d128_k16"; default:
    all).  A left-out variant makes the matching prefill call return
    HSA_ATTN_HIP_ERROR (not supported); the full build has every variant."""
    want = os.environ.get("HSA_ATTN_PREFILL_VARIANTS", "").strip()
    keep = {w.strip() for w in want.split(",") if w.strip()}
    out = []
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith(".hip"):
            continue
        if f.startswith("prefill_inst_") and keep and f[len("prefill_inst_"):-4] not in keep:
            continue
        out.append(os.path.join(CSRC, f))
    return out


def _variant_defines(srcs):
    defs = []
    for s in srcs:
        f = os.path.basename(s)
        if f.startswith("prefill_inst_"):
            defs.append("-DHSA_ATTN_HAVE_" + f[len("prefill_inst_"):-4].upper() + "=1")
    return defs


def _compile(src: str, defines=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *CXXFLAGS, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    # every symbol resolved at link time: a kernel whose host stub the host
    # pass left out would otherwise surface only when the library is loaded
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Builds libhsa_attn.so, and (debug=True) libhsa_attn_debug.so from the
    same sources with HSA_ATTN_DEBUG=1, plus the measurement probes."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    defines = _variant_defines(srcs)
    # slowest units first so the pool stays busy
    order = sorted(srcs, key=lambda s: not os.path.basename(s).startswith("prefill_inst_"))
    tasks = [(s, tuple(defines), BUILD) for s in order]
    if debug:
        os.makedirs(DEBUG_BUILD, exist_ok=True)
        tasks += [(s, tuple(defines) + ("-DHSA_ATTN_DEBUG=1",), DEBUG_BUILD) for s in order]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda t: _compile(*t), tasks))
    _link(objs[:len(order)], LIB)
    if debug:
        _link(objs[len(order):], DEBUG_LIB)
    tmp = STREAM_LIB + ".tmp"
    cmd = [hipcc(), *CXXFLAGS, "-shared", "-o", tmp, STREAM_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, STREAM_LIB)
    tmp = OVERLAP_EXE + ".tmp"
    cmd = [hipcc(), *CXXFLAGS, "-o", tmp, OVERLAP_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OVERLAP_EXE)
    if verbose:
        print(f"built {LIB}{', ' + DEBUG_LIB if debug else ''}, {STREAM_LIB} and {OVERLAP_EXE}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
