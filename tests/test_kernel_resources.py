"""Every kernel of the library runs without scratch memory (register spills).

The scan kernels count their own vector-memory operations in explicit waits,
so a spill there would break their accounting (their launchers also refuse a
build that spills); elsewhere a spill is hidden per-lane memory traffic.  The
check compiles each HIP source for gfx950 to assembly, with the library's own
flags, and reads the private segment size the compiler records for every
kernel.  No GPU is needed.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from selective_state_space_14_amd import build as hip_build

HIP_SOURCES = [s for s in hip_build.SOURCES if s.endswith(".hip")]


def _kernel_scratch(src: str, out_dir: str) -> dict:
    asm = os.path.join(out_dir, src + ".s")
    flags = [f for f in hip_build.CFLAGS if f not in ("-fPIC", "-Wall")]
    cmd = [hip_build.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(hip_build.CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-2000:]}"
    text = open(asm).read()
    # kernel metadata: one block per kernel with .name and .private_segment_fixed_size
    out = {}
    for block in re.split(r"\n  - \.", text.split("amdhsa.kernels:", 1)[1]):   # one per kernel
        name = re.search(r"\.name:\s+(\S+)", block)
        size = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        if name and size:
            out[name.group(1)] = int(size.group(1))
    return out


@pytest.mark.skipif(not (os.path.exists(hip_build.HIPCC) or shutil.which("hipcc")), reason="hipcc not found")
def test_no_kernel_uses_scratch(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        per_src = dict(zip(HIP_SOURCES, ex.map(lambda s: _kernel_scratch(s, str(tmp_path)), HIP_SOURCES)))
    kernels = {k: v for d in per_src.values() for k, v in d.items()}
    assert all(per_src.values()), {s: len(d) for s, d in per_src.items()}
    assert len(kernels) >= 100, len(kernels)   # every instantiation was read
    # the backward chunk kernel at every state size, N = 128 included
    for n in (16, 32, 64, 128):
        assert any(re.search(rf"ssd_bwd_chunk_kernel.*Li{n}E", k) for k in kernels), n
    spilled = {k: v for k, v in kernels.items() if v != 0}
    assert not spilled, spilled
