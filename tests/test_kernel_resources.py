"""Resource use of the gfx950 kernel, read from the compiler's own assembly
output for this source (hipcc --cuda-device-only -S): no VGPR spills, no
scratch (private segment) memory, LDS within the 160 KiB of a compute unit.
Scratch is not only slower inside the loop: a kernel that needs it pays
for its set-up at every launch."""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from block_scaled_fp4_group_amd import _build


def _kernel_metadata():
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        flags = [f for f in _build.FLAGS if f not in ("-fPIC", "-shared")]
        cmd = [_build.HIPCC, *flags, "-I" + _build.INCLUDE, _build.SRC, "--cuda-device-only", "-S", "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            pytest.fail("hipcc failed:\n" + res.stderr[-2000:])
        text = open(out).read()
    meta = {}
    for key in ("vgpr_spill_count", "private_segment_fixed_size", "group_segment_fixed_size", "vgpr_count"):
        m = re.findall(r"\.%s:\s+(\d+)" % key, text)
        assert m, "no %s in the kernel metadata" % key
        meta[key] = max(int(x) for x in m)
    return meta


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc not installed")
def test_kernel_uses_no_scratch_and_fits_lds():
    meta = _kernel_metadata()
    assert meta["vgpr_spill_count"] == 0, meta
    assert meta["private_segment_fixed_size"] == 0, meta
    assert meta["group_segment_fixed_size"] <= 160 * 1024, meta
    assert meta["vgpr_count"] <= 256, meta
