"""Every kernel instantiation compiles for gfx950 without register spills
(CPU only: runs hipcc's resource report on each translation unit)."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from row_normalization_persistent_amd import build as B


def _report(src):
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(B.CSRC, src), "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return src, r.stderr


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                    reason="hipcc not available")
def test_no_kernel_spills_registers():
    with cf.ThreadPoolExecutor(max_workers=len(B.SOURCES)) as ex:
        reports = list(ex.map(_report, B.SOURCES + B.CEILING_SOURCES))
    kernels = 0
    for src, text in reports:
        name = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                kernels += 1
                continue
            m = re.search(r"(VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
            if m and int(m.group(2)) != 0:
                pytest.fail(f"{src}: {name} has {m.group(1)} = {m.group(2)}")
    assert kernels > 100
