"""Register, scratch and LDS use of every kernel instance, from the
compiler's resource remarks (device-only compile for gfx950, no GPU needed).

Every instance keeps its state in registers (no scratch), except the
four-block (33-64 heads per KV head) matrix-path instances, which spill a
little by design and are only bounded. Scratch in the others once came from
compiler artefacts (the workgroup's unit range pinned in private memory and
reloaded behind a full memory wait at every piece; a hoisted pair of 64-bit
new-row pointers; sub-batch loads hoisted across an unrolled 256-dim tile),
not from real register pressure, so any scratch there is a regression to look
at. The instance counts pin the set of instances each file builds.
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from gqa_kv_cache_decode_amd import build

# Upper bound of the four-block matrix instances' spills (bytes per lane).
MAX_SPILL_FOUR_BLOCK = 256
LDS_BYTES = 160 * 1024  # per compute unit on gfx950
MAX_VGPRS = 256          # architected VGPRs a wave can address (occupancy aside)


SOURCES = ["decode_matrix.hip", "decode_stream.hip", "decode_vector.hip", "decode_vector_paged.hip",
           "decode_vector_multi.hip", "decode_vector_multi_paged.hip", "merge_partials.hip", "kv_append.hip",
           "fold_heads.hip", "linear.hip", "read_bandwidth.hip"]


@pytest.fixture(scope="module")
def remarks():
    """Resource remarks of every source, compiled in parallel once."""
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        return dict(zip(SOURCES, ex.map(lambda src: _resources(cc, src), SOURCES)))


def _resources(cc: str, source: str):
    cmd = [cc, "-x", "hip", *build.COMMON_FLAGS, "-I", build.CSRC, "--cuda-device-only", "-c", "-o", "/dev/null",
           os.path.join(build.CSRC, source), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    out, name = {}, None
    keys = {"VGPRs": "vgprs", "ScratchSize [bytes/lane]": "scratch", "LDS Size [bytes/block]": "lds"}
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        for key, field in keys.items():
            m = re.search(re.escape(key) + r": (\d+)", line)
            if m and name:
                out[name][field] = int(m.group(1))
    return out


def _check_common(inst):
    for name, r in inst.items():
        assert r["vgprs"] <= MAX_VGPRS, f"{name}: {r['vgprs']} VGPRs"
        assert r["lds"] <= LDS_BYTES, f"{name}: {r['lds']} bytes of LDS"


def test_matrix_kernel_instances_use_no_scratch_up_to_32_heads(remarks):
    res = remarks["decode_matrix.hip"]
    inst = {k: v for k, v in res.items() if "decode_matrix_kernel" in k}
    assert len(inst) == 18, sorted(inst)  # NB in {1, 2, 4} x fused / paged / causal forms
    _check_common(inst)
    for name, r in inst.items():
        nb = int(re.search(r"decode_matrix_kernelILi(\d+)E", name).group(1))
        if nb <= 2:
            assert r["scratch"] == 0, f"{name}: {r['scratch']} bytes of scratch per lane"
        else:
            assert r["scratch"] <= MAX_SPILL_FOUR_BLOCK, f"{name}: {r['scratch']} bytes of scratch per lane"


def test_stream_kernel_instances_use_no_scratch(remarks):
    res = remarks["decode_stream.hip"]
    inst = {k: v for k, v in res.items() if "decode_stream_kernel" in k}
    # fused x paged x causal x one, two or four head blocks, and the fused / unfused contiguous
    # one-token instances with split segments merged by their parts at the end of the launch
    assert len(inst) == 30, sorted(inst)
    _check_common(inst)
    for name, r in inst.items():
        assert r["scratch"] == 0, f"{name}: {r['scratch']} bytes of scratch per lane"
        # one workgroup per compute unit: the ring fills most of the LDS
        assert r["lds"] > LDS_BYTES // 2, f"{name}: {r['lds']} bytes of LDS"


@pytest.mark.parametrize("source,count", [("decode_vector.hip", 80), ("decode_vector_paged.hip", 80),
                                          ("decode_vector_multi.hip", 40), ("decode_vector_multi_paged.hip", 40)])
def test_vector_kernel_instances_use_no_scratch(remarks, source, count):
    # every element type, head dim (16 .. 256) and head block, fused or not
    res = remarks[source]
    inst = {k: v for k, v in res.items() if "decode_vector_kernel" in k}
    assert len(inst) == count, sorted(inst)
    _check_common(inst)
    for name, r in inst.items():
        assert r["scratch"] == 0, f"{name}: {r['scratch']} bytes of scratch per lane"


@pytest.mark.parametrize("source", ["merge_partials.hip", "kv_append.hip", "fold_heads.hip", "linear.hip",
                                    "read_bandwidth.hip"])
def test_other_kernels_use_no_scratch(remarks, source):
    res = remarks[source]
    assert res, f"no kernels found in {source}"
    _check_common(res)
    for name, r in res.items():
        assert r["scratch"] == 0, f"{name}: {r['scratch']} bytes of scratch per lane"
