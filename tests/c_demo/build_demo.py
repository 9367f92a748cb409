"""Compile decode_demo.c, a plain C consumer of libkvdecode, next to this file.

It links against the in-tree libkvdecode.so (found at run time relative to the
executable) and the HIP runtime, and is host code only: gcc builds it.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_demo.c")
EXE = os.path.join(HERE, "decode_demo")
LIBDIR = os.path.join(ROOT, "decode_attention_paged_04_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc")
    if cc is None:
        raise RuntimeError("gcc is needed to build the C consumer")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", EXE + ".tmp",
           "-L", LIBDIR, "-lkvdecode", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../decode_attention_paged_04_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
