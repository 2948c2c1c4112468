"""Every kernel of the library compiles for gfx950 without private (scratch)
memory: no vector-register spills and no stack objects. A kernel that uses
scratch reads and writes it through the same memory path as the state tiles,
so the HBM bytes would exceed the algorithmic bytes the benchmark reports.
(Scalar registers a kernel spills go to lanes of a vector register, with no
memory traffic, while its scratch size stays 0.) Runs on the CPU (hipcc
cross-compiles, device code only, with the library's own flags) and reads the
compiler's per-kernel resource remarks."""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from recurrent_state_storage_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not installed")

KERNEL_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _remarks(src):
    out = os.path.join("/tmp", f"rss_res_{os.getpid()}_{os.path.splitext(src)[0]}.o")
    cmd = [build.HIPCC, *build.FLAGS, *build.SOURCE_FLAGS.get(src, []), "-x", "hip", "-c",
           "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if os.path.exists(out):
        os.remove(out)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


def test_no_kernel_uses_scratch():
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        texts = dict(zip(KERNEL_SOURCES, ex.map(_remarks, KERNEL_SOURCES)))
    kernels = 0
    bad = []
    for src, text in texts.items():
        name = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                kernels += 1
                continue
            m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
            if m and int(m.group(2)) != 0:
                bad.append(f"{src}: {name}: {m.group(1)} = {m.group(2)}")
    assert kernels > 100, f"only {kernels} kernel remarks parsed"
    assert not bad, "\n".join(bad)
