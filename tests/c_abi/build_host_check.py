"""Build the host-only, sanitizer-instrumented check of the C ABI.

rss_api.cpp (validation, binding, sizing, call order) and abi_host_check.cpp
(its driver, with stub kernel launchers) are compiled for the host only, with
AddressSanitizer and UndefinedBehaviorSanitizer (errors not recoverable), into
tests/c_abi/abi_host_check. No GPU code is built and no GPU is needed to run it.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "abi_host_check")
SOURCES = [os.path.join(ROOT, "recurrent_state_storage_amd", "csrc", "rss_api.cpp"),
           os.path.join(HERE, "abi_host_check.cpp")]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# host-only sanitizers: every sanitizer flag applies to the host compilation
SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer", *SAN, f"-I{os.path.join(ROOT, 'include')}", *SOURCES, *SAN,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host check build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
