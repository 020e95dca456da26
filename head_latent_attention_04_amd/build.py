"""Build the MLA HIP library (libmla.so) in-tree for gfx950 with hipcc.

    python -m head_latent_attention_04_amd.build

Every HIP source under csrc/ is compiled to an object file, then all are linked into one
shared library next to this file. The measurement probe under probe/ (not part of the attention
path; bench.py's mfma_ceiling workload runs it) is built into a library of its own,
libmla_probe.so. Packed-FP32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
PROBE_SRC = os.path.join(PKG, "probe", "mfma_rate.hip")
PROBE_LIB = os.path.join(PKG, "libmla_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources, and {PROBE_LIB}")
    return LIB


def build_probe() -> str:
    """The MFMA-rate probe as its own shared library (bench.py --workload mfma_ceiling)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *common_flags(), "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime (preloaded into an uninstrumented host process)."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("AddressSanitizer runtime not found next to hipcc")
    return hits[-1]


def build_host_asan(out_dir: str) -> str:
    """The library with its host-side C-ABI layer (argument validation, workspace layout, launch
    set-up) built under AddressSanitizer; device code and the other objects are the regular build's.
    Returns the path of the shared library written to out_dir."""
    os.makedirs(out_dir, exist_ok=True)
    api = os.path.join(CSRC, "mla_api.hip")
    others = [s for s in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) if s != api]
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in others]
    if not all(os.path.exists(o) for o in objs):
        os.makedirs(BUILD, exist_ok=True)
        with cf.ThreadPoolExecutor(max_workers=min(8, len(others))) as ex:
            objs = list(ex.map(_compile, others))
    api_obj = os.path.join(out_dir, "mla_api_asan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [hipcc(), *common_flags(), "-O1", "-g", *san, "-c", api, "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    lib = os.path.join(out_dir, "libmla_asan.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", "-o", lib, api_obj, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return lib


if __name__ == "__main__":
    build()
