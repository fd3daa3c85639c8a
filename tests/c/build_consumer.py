"""Build the plain C consumer of the C ABI (tests/c/abi_rank_share) on the host.

Compiled with gcc as C99 against include/spattn.h and HIP's C runtime API and
linked to the in-tree libspattn.so (found at run time through an rpath
relative to the binary).  Called by the graft entry's build() after the
library; the GPU test that runs the binary does not build it.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_rank_share.c")
EXE = os.path.join(HERE, "abi_rank_share")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = EXE) -> list[str]:
    cc = os.environ.get("CC", shutil.which("gcc") or "cc")
    return [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", out,
            f"-L{os.path.join(ROOT, 'sequence_dit_attention_amd')}", "-lspattn", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
            "-Wl,-rpath,$ORIGIN/../../sequence_dit_attention_amd", f"-Wl,-rpath,{ROCM}/lib"]


def build(verbose: bool = False) -> str:
    r = subprocess.run(command(), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C consumer build failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {EXE}")
    return EXE
