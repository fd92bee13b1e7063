"""The spread merge of split segments (GQA_MERGE_SPREAD), against the fp64 oracle.

With the spread merge the stream kernel publishes every part of a split
segment and, at the end of the launch, each part merges its own slice of the
segment's heads once all parts have published; slices of parts that ended
before every workgroup had started (grids larger than the chip holds at once)
are merged by the workgroup that started last. The launch generation and the
flags live in the workspace's stamp region and are never reset.

Covered: the headline and 32-head shapes at grid sizes from one workgroup to
more than the chip holds (so that the orphaned slices and their sweep run),
bit-for-bit repeatability on one workspace across calls (the generation
advances, the arithmetic of a head depends only on its part count), the fused
step over several steps, and the edge shapes of the one-token tests.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_counters_zero, assert_parity, stamp_words, to_dev, to_host_bits, torch_dtype
from gqa_kv_cache_decode_amd import api
from gqa_kv_cache_decode_amd.workloads import WORKLOADS
from test_decode_gpu import EDGE, Problem
from test_step_gpu import StepProblem

pytestmark = pytest.mark.gpu

SPREAD = api.PATH_MATRIX | api.MERGE_SPREAD


def _workload_problem(oracle_mod, name):
    wl = WORKLOADS[name]
    pb = Problem(oracle_mod, seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=wl.lens,
                 dtype=wl.dtype)
    pb.append()
    return pb


def _run(pb, q_dev, ws, wgs, path=SPREAD):
    max_len = int(pb.lens_h.max())
    out = torch.empty(pb.b, pb.h, pb.d, dtype=torch_dtype(pb.dtype), device="cuda")
    api.decode_attention(out, q_dev, pb.kc, pb.vc, pb.lens, max_len, pb.scale, ws, path=path, workgroups=wgs)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["llama3_70b_gqa_bf16", "mqa_bf16", "mha_long_bf16_g1", "qwen25_7b_gqa_bf16"])
def test_spread_workloads_and_grids(gpu_lib, oracle_mod, name):
    print(f"spread merge: {name}", flush=True)
    pb = _workload_problem(oracle_mod, name)
    q = pb.query()
    ref = pb.oracle_attention(q)
    q_dev = to_dev(q)
    ws = api.make_workspace(pb.b, pb.h, pb.g, pb.d, pb.d, int(pb.lens_h.max()), torch_dtype(pb.dtype), "cuda")
    calls = 0
    for wgs in (0, 1, 7, 128, 2048):
        print(f"  workgroups={wgs}", flush=True)
        out = _run(pb, q_dev, ws, wgs)
        calls += 1
        assert_parity(out, ref, pb.dtype, f"{name} workgroups={wgs}")
        assert_counters_zero(ws, pb.b, pb.h)
        # one generation per call; the last workgroup to start published it
        assert stamp_words(ws) == (calls, calls)


@pytest.mark.parametrize("name,wgs", [("mqa_bf16", 0), ("mqa_bf16", 2048), ("llama3_70b_gqa_bf16", 1500)])
def test_spread_repeatable_bits(gpu_lib, oracle_mod, name, wgs):
    # which workgroup merges a head (its own part, or the sweep when the part
    # ended before every workgroup had started) changes from call to call;
    # the bits do not
    pb = _workload_problem(oracle_mod, name)
    q_dev = to_dev(pb.query())
    ws = api.make_workspace(pb.b, pb.h, pb.g, pb.d, pb.d, int(pb.lens_h.max()), torch_dtype(pb.dtype), "cuda")
    first = to_host_bits(_run(pb, q_dev, ws, wgs)).view(np.uint16)
    for _ in range(3):
        again = to_host_bits(_run(pb, q_dev, ws, wgs)).view(np.uint16)
        assert np.array_equal(first, again)
    # a fresh workspace (generation restarting at one) gives the same bits
    ws2 = api.make_workspace(pb.b, pb.h, pb.g, pb.d, pb.d, int(pb.lens_h.max()), torch_dtype(pb.dtype), "cuda")
    assert np.array_equal(first, to_host_bits(_run(pb, q_dev, ws2, wgs)).view(np.uint16))


@pytest.mark.parametrize("b,h,g,d,cap,lens,dtype", [e for e in EDGE if e[6] == "bf16" and e[3] == 128
                                                     and 3 <= e[1] // e[2] <= 64 and e[0] <= 64])
def test_spread_edge_shapes(gpu_lib, oracle_mod, b, h, g, d, cap, lens, dtype):
    pb = Problem(oracle_mod, seed=77 + h + d, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype)
    q = pb.query()
    ref = pb.oracle_attention(q)
    for wgs in (0, 1, 3, 64, 2048):
        out, ws = pb.gpu_attention(q, path=SPREAD, wgs=wgs)
        assert_parity(out, ref, dtype, f"spread workgroups={wgs}")
        assert_counters_zero(ws, b, h)
        for s in range(b):
            if pb.lens_h[s] == 0:
                assert torch.count_nonzero(out[s].float()) == 0


@pytest.mark.parametrize("b,h,g,lens,wgs", [
    (8, 32, 1, [4096] * 8, 0),                 # the MQA step
    (5, 64, 2, [0, 31, 32, 500, 698], 37),      # 32 heads per KV head, ragged, an empty sequence
    (3, 48, 1, [1, 333, 1000], 2048),           # 48 heads: two folding waves of 32, more parts than the chip holds
])
def test_spread_fused_steps(gpu_lib, oracle_mod, b, h, g, lens, wgs):
    cap = max(lens) + 8
    pb = StepProblem(oracle_mod, seed=311 + h, b=b, h=h, g=g, d=128, cap=cap, lens=lens, dtype="bf16")
    for step in range(3):
        print(f"spread fused step b={b} h={h} g={g} workgroups={wgs} step {step}", flush=True)
        got, ref = pb.step(step, path=SPREAD, wgs=wgs)
        assert_parity(got, ref, "bf16", f"step {step}")
        pb.check_state()
