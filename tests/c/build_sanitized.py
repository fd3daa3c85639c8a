"""Build the host-sanitized variant of libspattn.so for the CPU validation tests.

capi.cpp -- every argument check, the overflow arithmetic, the 128-bit bounds
and the grid checks -- is compiled host-only with AddressSanitizer and
UndefinedBehaviorSanitizer (no recovery: the first report aborts) and linked
with the kernel objects of the last library build (their device code is not
instrumented; GPU sanitizers are not used).  The result is
sequence_dit_attention_amd/_build/asan/libspattn_asan.so; the CPU test that
uses it runs the C-ABI validation cases against it in a child process with
the sanitizer runtime preloaded.  Nothing on the product path loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "sequence_dit_attention_amd")
BUILD = os.path.join(PKG, "_build")
OUT_DIR = os.path.join(BUILD, "asan")
LIB = os.path.join(OUT_DIR, "libspattn_asan.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or f"{ROCM}/bin/hipcc"
CLANGXX = f"{ROCM}/llvm/bin/clang++"
KERNEL_OBJS = ["attn_bf16.hip.o", "attn_d128.hip.o", "attn_d512.hip.o", "attn_f32.hip.o", "pack.hip.o", "rope.hip.o"]


def runtime() -> str:
    """Path of the shared AddressSanitizer runtime to preload."""
    return subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    obj = os.path.join(OUT_DIR, "capi_asan.o")
    # Host pass only; each sanitizer flag is scoped to the host compilation.
    compile_cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip", "--cuda-host-only",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-c", os.path.join(PKG, "csrc", "capi.cpp"), "-o", obj]
    link_cmd = [CLANGXX, "-shared", "-shared-libsan", "-fsanitize=address,undefined", "-o", LIB, obj,
                *[os.path.join(BUILD, o) for o in KERNEL_OBJS], f"-L{ROCM}/lib", "-lamdhip64",
                f"-Wl,-rpath,{ROCM}/lib"]
    for cmd in (compile_cmd, link_cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB}")
    return LIB
