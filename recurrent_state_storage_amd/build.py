"""Compile librss.so for gfx950 in-tree with hipcc.

Objects go to recurrent_state_storage_amd/_build/, the library to
recurrent_state_storage_amd/librss.so (written to a temporary name, then
renamed, so a process that has the old library loaded keeps a valid file).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librss.so")

SOURCES = ["replay.hip", "flush.hip", "eager.hip", "gdn.hip", "calib.hip", "rss_api.cpp"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 (v_pk_*_f32) is kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Per-source flags. The replay kernels keep their few matrix-core accumulators
# (a verify's ring terms) in ordinary VGPRs: with AGPRs the verify with the
# committed-window fold needs 77 + 4 registers, one allocation granule past six
# wavefronts per SIMD; in VGPR form it needs 77. (The folds in the flush and
# delta-rule kernels, with 32 accumulators, are better off in AGPRs.)
SOURCE_FLAGS = {"replay.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link librss.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "rss_c_driver.cpp")
DRIVER = os.path.join(ROOT, "tests", "c_abi", "rss_c_driver")


def build_c_driver(verbose: bool = False) -> str:
    """Compile the plain C++ test caller of the C ABI (host code only), linked
    against librss.so with a relative run path, so it finds the in-tree library
    wherever the repository is copied."""
    tmp = DRIVER + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-Wall",
           f"-I{os.path.join(ROOT, 'include')}", DRIVER_SRC, f"-L{PKG}", "-lrss",
           "-Wl,-rpath,$ORIGIN/../../recurrent_state_storage_amd", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {DRIVER_SRC}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DRIVER)
    if verbose:
        print(f"built {DRIVER}")
    return DRIVER


if __name__ == "__main__":
    build(verbose=True)
    build_c_driver(verbose=True)
