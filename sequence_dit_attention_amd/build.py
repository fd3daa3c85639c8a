"""Build libspattn.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object in _build/ (in parallel) and
linked into sequence_dit_attention_amd/libspattn.so.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-file flags.  The head-size-64 attention kernel keeps every MFMA operand
# and result in VGPRs (the scores feed VALU softmax code; AGPR copies would
# cost more than they save); the head-size-128 kernel writes all its MFMAs as
# inline asm on VGPRs; the head-size-512 kernel keeps its O accumulators in
# AGPRs (the default MFMA form; its score MFMAs are inline asm on VGPRs).  None
# needs NaN canonicalisation before its max reductions.
EXTRA = {
    "attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true", "-fno-honor-nans"],
    "attn_d128.hip": ["-fno-honor-nans"],
    "attn_d512.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
