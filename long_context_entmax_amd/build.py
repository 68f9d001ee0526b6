"""Build the HIP library ``libentmax_attn.so`` in-tree with hipcc for gfx950.

``python -m long_context_entmax_amd.build`` compiles every source under ``csrc/``
(one object per file, in parallel) and links the shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libentmax_attn.so")
SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "prep.hip", "decode.hip", "dash.hip"]
ARCH = os.environ.get("ENTMAX_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
    # extra hipcc flags for tuning builds (e.g. -DENTMAX_HIST_WAVES64=4)
    *os.environ.get("ENTMAX_HIPCC_FLAGS", "").split(),
]


# per-source flags: the backward kernels convert matrix-core results to operands on every
# tile; with the results in VGPRs (not accumulation registers) no copy precedes each
# conversion, which at head_dim 128 (one wave per SIMD, every register in use) removes
# several hundred copies per tile
FILE_FLAGS = {
    "bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "dash.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")


def build(verbose: bool = False) -> str:
    """Compile and link; always rebuilds. Returns the library path."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    jobs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(bdir, s.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append((src, obj))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libentmax_attn.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
