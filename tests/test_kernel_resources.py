"""Register budgets of the device code, checked on the host: every HIP source
is compiled for gfx950 with the library's own flags and the compiler's
resource report must show no scratch memory and no VGPR spills for any
kernel. Scratch in a streaming kernel costs memory traffic per lane, and it
has crept in before through register pressure alone."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from decode_phase_attention_amd import build as B

SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def resources(src):
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-shared"], "--cuda-device-only", "-c",
           "-I", os.path.join(B.ROOT, "include"), os.path.join(B.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|VGPRs): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                    reason="no hipcc")
def test_no_scratch_and_no_spills():
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        reports = dict(zip(SOURCES, ex.map(resources, SOURCES)))
    assert all(reports.values()), "no kernels found in the resource report"
    names = set()
    for src, kernels in reports.items():
        for name, r in kernels.items():
            names.add(name)
            assert r.get("ScratchSize [bytes/lane]") == 0, (src, name, r)
            assert r.get("VGPRs Spill") == 0, (src, name, r)
            assert 0 < r.get("VGPRs", 0) <= 256, (src, name, r)
    # the lean kernels of both head types, at every schedule source
    for kind in ("lean_kernel", "lean_gqa_kernel"):
        assert sum(kind + "I" in n for n in names) == 12, kind
