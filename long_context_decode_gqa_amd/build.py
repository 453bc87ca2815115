"""Build libwmtp.so (HIP for gfx950) in-tree with hipcc.

`python -m long_context_decode_gqa_amd.build` compiles every source under
csrc/ into long_context_decode_gqa_amd/_lib/libwmtp.so.  The build always
recompiles (it is the "does it build" check); objects go to _build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
OBJ_DIR = os.path.join(ROOT, "_build", "wmtp")
LIB = os.path.join(OUT_DIR, "libwmtp.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable", "-Wno-unused-but-set-variable"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


UBSAN_LIB = os.path.join(ROOT, "_build", "ubsan", "libwmtp.so")


def build_host_ubsan(verbose: bool = False) -> str:
    """A variant of the library whose host code (the C ABI's checks and planners) carries the
    undefined-behaviour sanitizer, minimal runtime, aborting on the first report; the device code
    is the same.  For the CPU suite: WMTP_LIBRARY=<this path> python -m pytest tests -m "not gpu"."""
    build(verbose=False)                  # the device objects
    flags = ["-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fsanitize-minimal-runtime"]
    abi = os.path.join(CSRC, "wmtp_abi.cpp")
    obj = os.path.join(OBJ_DIR, "wmtp_abi.ubsan.o")
    cmd = [HIPCC, "-x", "hip", *COMMON, *flags, "-Xarch_host", "-fno-sanitize-recover=all", "-c", abi, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {abi}:\n{r.stderr}")
    objs = [os.path.join(OBJ_DIR, os.path.basename(src) + ".o") for src in sources() if src != abi] + [obj]
    res = subprocess.run([HIPCC, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    found = [os.path.join(d, f) for d, _, fs in os.walk(os.path.join(res, "lib")) for f in fs
             if f.startswith("libclang_rt.ubsan_minimal") and f.endswith(".so")]
    if not found:
        raise RuntimeError(f"no minimal UBSan runtime under {res}")
    rt_dir = os.path.dirname(found[0])
    os.makedirs(os.path.dirname(UBSAN_LIB), exist_ok=True)
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", *flags, "-shared-libsan", f"-Wl,-rpath,{rt_dir}",
           "-o", UBSAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {UBSAN_LIB}")
    return UBSAN_LIB


if __name__ == "__main__":
    if "--host-ubsan" in sys.argv[1:]:
        build_host_ubsan(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
