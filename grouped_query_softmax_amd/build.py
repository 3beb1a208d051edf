"""Build ``libgqa_attn.so`` in-tree with hipcc for gfx950.

Usage: ``python grouped_query_softmax_amd/build.py`` (run as a file: importing it through the
package would first load the library it builds), or ``build()`` from Python. Each source is
compiled to an object under ``_build/`` (parallel), then linked into the package directory.
Always recompiles: this is the "does it build" check as well as the build.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
from typing import List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgqa_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["gqa_attn_api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip", "fold.hip",
           "backward.hip", "keys.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs ROCm)")


# Per-file flags. The bf16 attention kernels assume finite (non-NaN) inputs: with NaN semantics
# relaxed, maxima of matrix-core results compile to v_max3_f32 without a canonicalising
# v_max_f32 per element. Infinities keep their meaning (masked scores are -inf).
FILE_FLAGS = {
    "prefill_bf16.hip": ["-fno-honor-nans"],
    # decode also keeps its matrix-core accumulators in ordinary VGPRs, so the occasional softmax
    # rescale of the output accumulators needs no accumulator-register copies
    "decode.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the backward's gradient accumulators are read by vector code between products (the
    # cross-wave sums); in accumulator registers the compiler copied them in and out around
    # every product
    "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, extra: List[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *extra, *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra_flags: Optional[List[str]] = None, verbose: bool = False) -> str:
    extra = list(extra_flags or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
