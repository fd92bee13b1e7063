"""GPU parity of the fused step (gqa_decode_step): append + attention in one launch.

After each step the caches and lengths must equal the oracle's append bit for
bit, and the output must meet the parity bar against the oracle's attention
over the cache including the appended token. Covers every workload, both
kernels and several grid sizes, appending into an empty sequence and into the
last free slot, a 32-step loop, and equivalence with the two-call sequence.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_counters_zero, assert_parity, to_dev, to_host_bits, torch_dtype
from gqa_kv_cache_decode_amd import api, inputs
from gqa_kv_cache_decode_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu


class StepProblem:
    def __init__(self, oracle_mod, *, seed, b, h, g, d, cap, lens, dtype, scale=None):
        self.b, self.h, self.g, self.d, self.cap, self.dtype = b, h, g, d, cap, dtype
        self.scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
        self.batch = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
        self.kc, self.vc = to_dev(self.batch.k_cache), to_dev(self.batch.v_cache)
        self.lens_h = self.batch.lens.copy()
        self.lens = torch.from_numpy(self.lens_h.copy()).cuda()
        self.oracle = oracle_mod
        self.ws = api.make_workspace(b, h, g, d, d, cap, torch_dtype(dtype), "cuda")

    def step(self, step, path=api.PATH_AUTO, wgs=0, rows=None):
        q = self.batch.q(step)
        kn, vn = self.batch.new_kv(step)
        out = torch.empty(self.b, self.h, self.d, dtype=torch_dtype(self.dtype), device="cuda")
        api.decode_step(out, to_dev(q), to_dev(kn), to_dev(vn), self.kc, self.vc, self.lens, int(self.lens_h.max()),
                        self.scale, self.ws, path=path, workgroups=wgs)
        torch.cuda.synchronize()
        self.oracle.kv_append(self.batch.k_cache, self.batch.v_cache, kn, vn, self.lens_h)
        if rows is None:
            ref = self.oracle.decode_attention(q, self.batch.k_cache, self.batch.v_cache, self.lens_h, self.scale)
            got = out
        else:
            sub = lambda a: np.ascontiguousarray(a[rows])
            ref = self.oracle.decode_attention(sub(q), sub(self.batch.k_cache), sub(self.batch.v_cache),
                                               sub(self.lens_h), self.scale)
            got = out[torch.from_numpy(rows).cuda()]
        return got, ref

    def check_state(self):
        assert np.array_equal(self.lens.cpu().numpy(), self.lens_h)
        assert np.array_equal(to_host_bits(self.kc).view(np.uint8), self.batch.k_cache.view(np.uint8))
        assert np.array_equal(to_host_bits(self.vc).view(np.uint8), self.batch.v_cache.view(np.uint8))
        assert_counters_zero(self.ws, self.b, self.h)  # tickets and the step's finish counter


def _workload(oracle_mod, name):
    wl = WORKLOADS[name]
    return StepProblem(oracle_mod, seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=wl.lens,
                       dtype=wl.dtype)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_step_workloads(gpu_lib, oracle_mod, name):
    print(f"fused step parity: {name}", flush=True)
    pb = _workload(oracle_mod, name)
    got, ref = pb.step(0)
    assert_parity(got, ref, pb.dtype, name)
    pb.check_state()


@pytest.mark.parametrize("path,wgs", [(api.PATH_MATRIX, 0), (api.PATH_MATRIX, 1), (api.PATH_MATRIX, 37),
                                      (api.PATH_MATRIX, 2048), (api.PATH_VECTOR, 0), (api.PATH_VECTOR, 3),
                                      (api.PATH_MATRIX | api.MERGE_KERNEL, 37),
                                      (api.PATH_MATRIX | api.MERGE_KERNEL, 2048),
                                      (api.PATH_VECTOR | api.MERGE_KERNEL, 3),
                                      (api.PATH_MATRIX | api.MERGE_INLINE, 2048)])
def test_step_paths_and_grids(gpu_lib, oracle_mod, path, wgs):
    pb = StepProblem(oracle_mod, seed=301, b=5, h=16, g=2, d=128, cap=700, lens=[0, 31, 32, 500, 698],
                     dtype="bf16")
    for step in range(2):
        got, ref = pb.step(step, path=path, wgs=wgs)
        assert_parity(got, ref, "bf16", f"path={path} workgroups={wgs} step={step}")
        pb.check_state()


@pytest.mark.parametrize("h,g,lens,wgs", [(32, 1, [0, 31, 32, 95], 0), (32, 1, [0, 31, 32, 95], 5),
                                          (40, 2, [70, 1, 64, 33], 0), (64, 2, [96, 97], 3)])
def test_step_wide_head_groups(gpu_lib, oracle_mod, h, g, lens, wgs):
    # 17 to 32 query heads per KV head (two MFMA column blocks), ragged tails
    # around the 32-position tiles, poisoned slots past every length
    print(f"wide head groups: h={h} g={g} lens={lens} workgroups={wgs}", flush=True)
    pb = StepProblem(oracle_mod, seed=320 + h + wgs, b=len(lens), h=h, g=g, d=128, cap=104, lens=lens, dtype="bf16")
    for step in range(4):
        merge = api.MERGE_KERNEL if step == 3 else api.MERGE_INLINE
        got, ref = pb.step(step, path=api.PATH_MATRIX | merge, wgs=wgs)
        assert_parity(got, ref, "bf16", f"step {step} merge={merge:#x}")
        pb.check_state()


@pytest.mark.parametrize("dtype,d,h,g", [("f32", 16, 4, 2), ("f32", 128, 8, 8), ("bf16", 64, 12, 3),
                                         ("bf16", 256, 4, 1), ("f32", 256, 6, 2)])
def test_step_vector_shapes(gpu_lib, oracle_mod, dtype, d, h, g):
    pb = StepProblem(oracle_mod, seed=302 + d, b=3, h=h, g=g, d=d, cap=70, lens=[0, 33, 68], dtype=dtype)
    for step in range(2):
        got, ref = pb.step(step)
        assert_parity(got, ref, dtype, f"step {step}")
        pb.check_state()


def test_step_into_empty_sequence_returns_new_value(gpu_lib, oracle_mod):
    # a sequence with nothing cached attends only to the appended token: out = v_new
    pb = StepProblem(oracle_mod, seed=303, b=2, h=8, g=2, d=128, cap=40, lens=[0, 0], dtype="bf16")
    got, ref = pb.step(0)
    assert_parity(got, ref, "bf16")
    _, vn = pb.batch.new_kv(0)
    want = inputs.bf16_bits_to_f32(np.repeat(vn, 4, axis=1)).astype(np.float64)
    np.testing.assert_allclose(inputs.bf16_bits_to_f32(to_host_bits(got)).astype(np.float64), want, atol=1e-2)
    pb.check_state()


def test_step_loop_32(gpu_lib, oracle_mod):
    wl = WORKLOADS["qwen25_7b_gqa_bf16"]
    print("fused step loop: qwen25_7b_gqa_bf16, 32 steps", flush=True)
    pb = _workload(oracle_mod, wl.name)
    for step in range(wl.steps):
        # every sequence and head against the oracle, and the caches, lengths
        # and counters, after every step
        got, ref = pb.step(step)
        assert_parity(got, ref, pb.dtype, f"step {step}")
        pb.check_state()
    assert int(pb.lens_h.min()) == int(pb.lens_h.max()) == 2080


def test_step_equals_two_calls(gpu_lib, oracle_mod):
    a = StepProblem(oracle_mod, seed=304, b=4, h=32, g=4, d=128, cap=600, lens=[1, 100, 333, 598], dtype="bf16")
    b = StepProblem(oracle_mod, seed=304, b=4, h=32, g=4, d=128, cap=600, lens=[1, 100, 333, 598], dtype="bf16")
    got_a, _ = a.step(0)
    q = b.batch.q(0)
    kn, vn = b.batch.new_kv(0)
    api.kv_append(b.kc, b.vc, to_dev(kn), to_dev(vn), b.lens, int(b.lens_h.max()))
    out = torch.empty_like(got_a)
    api.decode_attention(out, to_dev(q), b.kc, b.vc, b.lens, int(b.lens_h.max()) + 1, b.scale, b.ws)
    torch.cuda.synchronize()
    assert torch.equal(a.lens, b.lens)
    assert torch.equal(a.kc.view(torch.int16), b.kc.view(torch.int16))
    assert torch.equal(a.vc.view(torch.int16), b.vc.view(torch.int16))
    assert (got_a.float() - out.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("b,path,dtype,d", [(64, api.PATH_MATRIX, "bf16", 128), (65, api.PATH_MATRIX, "bf16", 128),
                                            (130, api.PATH_VECTOR, "f32", 32), (200, api.PATH_AUTO, "bf16", 64)])
def test_step_batch_sizes_around_64(gpu_lib, oracle_mod, b, path, dtype, d):
    # up to 64 sequences the kernels keep lens in registers and count the
    # workgroups out early; beyond that they read lens while walking
    lens = [(37 * s) % 150 for s in range(b)]
    pb = StepProblem(oracle_mod, seed=305 + b, b=b, h=8, g=2, d=d, cap=160, lens=lens, dtype=dtype)
    for step in range(3):
        got, ref = pb.step(step, path=path)
        assert_parity(got, ref, dtype, f"b={b} step={step}")
        pb.check_state()


def test_step_maximum_batch(gpu_lib, oracle_mod):
    # the largest batch: the last workgroup writes all 65535 grown lengths
    b = 65535
    lens = np.random.default_rng(7).integers(0, 3, size=b).tolist()
    pb = StepProblem(oracle_mod, seed=306, b=b, h=2, g=1, d=16, cap=5, lens=lens, dtype="f32")
    for step in range(2):
        got, ref = pb.step(step)
        assert_parity(got, ref, "f32", f"step {step}")
        pb.check_state()


def test_step_on_a_side_stream_equals_the_default_stream(gpu_lib, oracle_mod):
    # the binding launches on torch's current stream: inside a side stream's
    # context the step runs there (ordered after the inputs' copies by an
    # explicit wait) and gives the same bits as on the default stream
    a = StepProblem(oracle_mod, seed=307, b=3, h=32, g=2, d=128, cap=400, lens=[0, 129, 398], dtype="bf16")
    b = StepProblem(oracle_mod, seed=307, b=3, h=32, g=2, d=128, cap=400, lens=[0, 129, 398], dtype="bf16")
    got_a, ref = a.step(0)
    q = b.batch.q(0)
    kn, vn = b.batch.new_kv(0)
    qd, knd, vnd = to_dev(q), to_dev(kn), to_dev(vn)
    out = torch.empty(b.b, b.h, b.d, dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        api.decode_step(out, qd, knd, vnd, b.kc, b.vc, b.lens, int(b.lens_h.max()), b.scale, b.ws)
    side.synchronize()
    assert torch.equal(out.view(torch.int16), got_a.view(torch.int16))
    assert_parity(out, ref, "bf16", "side stream")
    b.oracle.kv_append(b.batch.k_cache, b.batch.v_cache, kn, vn, b.lens_h)
    b.check_state()
