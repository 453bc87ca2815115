"""Build the C program that drives libwmtp's C ABI without Python (tests/c_abi/decode_step.c).

`python -m tests.c_abi.build` (also run by the repository's build entry point after the
library) compiles it with the host C compiler against include/wmtp.h and the in-tree
libwmtp.so, into tests/c_abi/_bin/decode_step, with run paths to the library and to ROCm.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_step.c")
BIN = os.path.join(HERE, "_bin", "decode_step")
LIB_DIR = os.path.join(ROOT, "long_context_decode_gqa_amd", "_lib")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler (gcc) for tests/c_abi/decode_step.c")
    rel = os.path.relpath(LIB_DIR, os.path.dirname(BIN))
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", BIN,
           "-L", LIB_DIR, "-lwmtp", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {SRC} failed:\n{r.stderr}")
    if verbose:
        print(f"built {BIN}")
    return BIN


if __name__ == "__main__":
    build(verbose=True)
