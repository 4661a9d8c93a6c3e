"""Compile the plain-C consumer of libsmla.so (smla_c_bwd.c) next to its source.

It includes only include/smla.h and the HIP runtime's C API header, and links
the in-tree libsmla.so (found at run time through an rpath relative to the
binary) and libamdhip64.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "sparse_mla_attention_smla_amd")
BIN = os.path.join(HERE, "smla_c_bwd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C-ABI consumer")
    rel = os.path.relpath(PKG, HERE)
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "smla_c_bwd.c"), "-o", BIN + ".tmp",
           "-L", PKG, "-lsmla", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C consumer build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
