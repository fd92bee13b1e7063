"""Register and scratch use of the matrix decode kernel, from the compiler's
resource remarks (device-only compile for gfx950, no GPU needed).

The one- and two-block instances (up to 32 heads per KV group) keep all their
state in registers. Scratch there once came from a compiler artefact (the
workgroup's unit range pinned in private memory, reloaded behind a full
memory wait at every piece), not from register pressure, so any scratch in
these instances is a regression to look at. The four-block (33-64 heads)
instances spill a little by design; they are only bounded.
"""
import os
import re
import subprocess

import pytest

from gqa_kv_cache_decode_amd import build

# Upper bound of the four-block instances' spills (bytes per lane).
MAX_SPILL_FOUR_BLOCK = 256


def _resources(source: str):
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    cmd = [cc, "-x", "hip", *build.COMMON_FLAGS, "-I", build.CSRC, "--cuda-device-only", "-c", "-o", "/dev/null",
           source, "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    out, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


def test_matrix_kernel_instances_use_no_scratch_up_to_32_heads():
    scratch = _resources(os.path.join(build.CSRC, "decode_matrix.hip"))
    inst = {k: v for k, v in scratch.items() if "decode_matrix_kernel" in k}
    assert len(inst) == 18, sorted(inst)  # NB in {1, 2, 4} x fused / paged / causal forms
    for name, bytes_per_lane in inst.items():
        nb = int(re.search(r"decode_matrix_kernelILi(\d+)E", name).group(1))
        if nb <= 2:
            assert bytes_per_lane == 0, f"{name}: {bytes_per_lane} bytes of scratch per lane"
        else:
            assert bytes_per_lane <= MAX_SPILL_FOUR_BLOCK, f"{name}: {bytes_per_lane} bytes of scratch per lane"
