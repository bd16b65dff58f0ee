"""Every kernel of the library keeps its state in registers and LDS.

The short-row and split finishers hold their survivors in register arrays
indexed by unrolled loops; a change that defeats the unrolling (a loop exit
in a loop of ballots, say) makes the compiler move those arrays to scratch
memory without any error, and register spills do the same. This test
compiles each source for gfx950 the way the library build does (device code
only, to assembly) and reads the kernel descriptors: no kernel may use
private (scratch) memory or spill vector registers. Scalar registers may
spill (into vector-register lanes, not memory). CPU only: hipcc
cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from exact_row_top_fp32_amd import build

SOURCES = {os.path.basename(s): s for s in build.SOURCES}


def kernel_resources(source: str, tmp_path) -> dict:
    out = tmp_path / (os.path.basename(source) + ".s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", build.INCLUDE, source, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    kernels = {}
    # the metadata lists each kernel's fields in one block, .name among them
    for block in re.split(r"\n\s*- \.", text.split("amdhsa.kernels:", 1)[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        fields = {}
        for key in ("private_segment_fixed_size", "vgpr_spill_count", "sgpr_spill_count", "vgpr_count"):
            m = re.search(r"\." + key + r":\s+(\d+)", block)
            fields[key] = int(m.group(1)) if m else None
        kernels[name.group(1)] = fields
    return kernels


@pytest.mark.parametrize("source", sorted(SOURCES))
def test_no_scratch_and_no_vector_spills(source, tmp_path):
    kernels = kernel_resources(SOURCES[source], tmp_path)
    assert kernels, "no kernel descriptors found"
    bad = {k: v for k, v in kernels.items()
           if v["private_segment_fixed_size"] != 0 or v["vgpr_spill_count"] != 0}
    assert not bad, f"kernels with scratch memory or vector spills: {bad}"
