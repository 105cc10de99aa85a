"""Compile the gfx950 HIP library in-tree: mla_latent_kv_10_amd/libmla_mi355x.so.

Usage: python -m mla_latent_kv_10_amd.build  (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmla_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# The same library with the split kernel built to wait for every tile's loads
# right after issuing them (MLA_DRAIN_PIPELINE): the LDS race check compares
# its outputs with the pipelined library's, bit for bit.
DRAIN_LIB_PATH = os.path.join(HERE, "libmla_mi355x_drain.so")
SOURCES = ["mla_abi.cpp", "mla_metadata.hip", "mla_decode.hip", "mla_combine.hip", "mla_quantize.hip", "mla_absorb.hip",
           "mla_probe.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
    # packed fp32 VALU forms are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# The decode kernel keeps MFMA accumulators of the score tile in VGPRs
# (VGPR form) and pins the output accumulator to AGPRs with inline asm.
# Kernel-argument preload (SGPRs filled at dispatch; the count is in arguments)
# for the combine (one leading pointer) and the schedule kernel (nine
# scalars). The split kernel does not use it: preloading its schedule pointer
# measured slower.
EXTRA_FLAGS = {
    "mla_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "mla_combine.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=1"],
    "mla_metadata.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=9"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link the shared library. Returns its path."""
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="mla_build_")
    try:
        def compile_one(job):
            src, tag, defs = job
            obj = os.path.join(tmp, os.path.basename(src) + tag + ".o")
            cmd = [hipcc, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), *defs, "-x", "hip", "-c",
                   os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            if verbose:
                print(f"compiled {src}{tag}", flush=True)
            return obj

        jobs_list = [(src, "", []) for src in SOURCES] + [("mla_decode.hip", ".drain", ["-DMLA_DRAIN_PIPELINE"])]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, jobs_list))
        main_objs = objs[:len(SOURCES)]
        drain_objs = [objs[-1] if src == "mla_decode.hip" else o for src, o in zip(SOURCES, main_objs)]
        for path, parts in ((LIB_PATH, main_objs), (DRAIN_LIB_PATH, drain_objs)):
            out_tmp = path + ".tmp"
            cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *parts, "-o", out_tmp]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            os.replace(out_tmp, path)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if verbose:
        print(f"built {LIB_PATH}", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
