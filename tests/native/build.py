"""Builds the plain C caller of the C-ABI library (tests/native/pre_attn_caller) against the
in-tree libdit.so, with gcc and the HIP runtime's C API."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "diffusion_transformer_adaln_rmsnorm_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BINARY = os.path.join(HERE, "pre_attn_caller")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "pre_attn_caller.c"), f"-L{PKG}", "-ldit",
           f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../diffusion_transformer_adaln_rmsnorm_amd",
           f"-Wl,-rpath,{ROCM}/lib", "-o", BINARY + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY


if __name__ == "__main__":
    build(verbose=True)
