"""Every kernel compiles without register spills (CPU only: hipcc
cross-compiles for gfx950 and reports each kernel's resources).

A spill puts scratch loads and stores into a kernel; in the grouped GEMM's
K loop they cost more than everything else (a one-line change in an
epilogue once made the backward's dH / dX GEMM spill 140 bytes a lane and
run 60% slower).  The forward-and-keep GEMM (phase 4) keeps one value of
its prologue in scratch, outside the loops."""
import os
import re
import subprocess

import pytest

from top_routing_expert_softmax_amd import build as B

# kernel name pattern -> largest scratch (bytes per lane) allowed; every
# other kernel: none
LIMITS = [
    (r"gemm_big_kernelILi4E", 8),
]


def resources(src):
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-c", os.path.join(B.CSRC, src),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", [os.path.basename(p) for p in B.sources()])
def test_kernels_do_not_spill(src):
    with open(os.path.join(B.CSRC, src)) as fh:
        if "__global__" not in fh.read():
            pytest.skip("no kernels in this source")
    res = resources(src)
    assert res, f"no kernels reported for {src}"
    for name, scratch in res.items():
        limit = next((lim for pat, lim in LIMITS if re.search(pat, name)), 0)
        assert scratch <= limit, f"{name}: {scratch} bytes of scratch a lane"
