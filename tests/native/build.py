"""Build the native C caller (tests/native/decode_caller.c) against the
in-tree libdecode_attn.so and the HIP runtime, with the host C compiler.

    python tests/native/build.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "paged_kv_cache_471_amd")
SRC = os.path.join(HERE, "decode_caller.c")
EXE = os.path.join(HERE, "decode_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the native caller")
    rocm_lib = os.path.join(ROCM, "lib")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", EXE + ".tmp",
           "-L", PKG, "-ldecode_attn", "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_471_amd", "-L", rocm_lib, "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"native caller build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    if verbose:
        print(f"built {EXE}")
    return EXE


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
