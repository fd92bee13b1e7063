"""GPU parity of multi-token decode (gqa_kv_append_multi, gqa_decode_attention_multi,
gqa_decode_step_multi) against the fp64 oracle.

n new tokens per sequence sit at positions L .. L + n - 1; token r attends the
cache and the new tokens up to itself. The kernels run the n * h/g query rows
of a KV group together (on the matrix cores, or a head block at a time on the
vector path), one K/V read for all of them. Checked: outputs to the decode
parity bar (every token, every head) at group sizes that take one, two and
four 16-row MFMA blocks, the vector path (fp32, other head dims, fewer than
three or more than 64 virtual heads), lengths whose new tokens straddle a
tile boundary or fill an empty cache, and the split merge done by a second
launch; the appended rows bit for bit; n = 1 equal bit for bit to the
one-token call; a multi-step loop; the Llama-3-70B shape.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from gqa_kv_cache_decode_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

CASES = [
    # b, h, g, n, pre-append lengths[, dtype, d]
    (3, 64, 8, 2, [0, 30, 300]),        # 16 virtual heads: one MFMA block, 8 waves
    (3, 64, 8, 4, [1, 29, 511]),        # 32: two blocks
    (2, 64, 8, 8, [5, 700]),            # 64: four blocks
    (4, 28, 4, 3, [0, 62, 63, 200]),    # 21: G = 7
    (2, 32, 1, 2, [900, 3000]),         # MQA, 64 virtual heads, split merge by a second launch
    (3, 8, 8, 4, [3, 33, 97]),          # MHA-shaped (G = 1), 4 virtual heads
    (2, 16, 4, 1, [40, 1000]),          # n = 1
    (3, 8, 8, 2, [3, 33, 97]),          # 2 virtual heads: the vector path
    (2, 72, 8, 8, [64, 300]),           # 72 virtual heads (> 64): the vector path, head blocks of 8
    (3, 8, 4, 3, [0, 31, 100], "f32", 16),    # fp32 (vector path), the tiny shape's head dim
    (2, 16, 4, 4, [10, 200], "bf16", 64),     # bf16, d = 64 (vector path)
    (2, 12, 3, 2, [70, 33], "f32", 256),      # fp32, d = 256
]


def _unpack(case):
    b, h, g, n, lens = case[:5]
    dtype = case[5] if len(case) > 5 else "bf16"
    d = case[6] if len(case) > 6 else 128
    return b, h, g, n, lens, dtype, d


def _draw(rng, shape, dtype="bf16"):
    x = rng.standard_normal(shape).astype(np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


class MultiProblem:
    def __init__(self, b, h, g, n, lens, seed, steps=1, dtype="bf16", d=128):
        self.b, self.h, self.g, self.n, self.d, self.dtype = b, h, g, n, d, dtype
        self.tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        cap = max(lens) + n * steps + 8
        self.batch = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
        self.cap = cap
        self.rng = np.random.default_rng(seed)
        self.scale = float(np.float32(1.0 / np.sqrt(d)))
        self.kc, self.vc = to_dev(self.batch.k_cache), to_dev(self.batch.v_cache)
        self.lens = torch.from_numpy(self.batch.lens.copy()).cuda()
        self.kc_h, self.vc_h, self.lens_h = self.batch.k_cache.copy(), self.batch.v_cache.copy(), self.batch.lens.copy()
        self.ws = api.make_multi_workspace(b, n, h, g, d, d, self.tdt, "cuda")

    def draw_step(self):
        return (_draw(self.rng, (self.b, self.n, self.h, self.d), self.dtype),
                _draw(self.rng, (self.b, self.n, self.g, self.d), self.dtype),
                _draw(self.rng, (self.b, self.n, self.g, self.d), self.dtype))


def _id(c):
    b, h, g, n, lens, dtype, d = _unpack(c)
    return f"h{h}g{g}n{n}" + ("" if (dtype, d) == ("bf16", 128) else f"-{dtype}-d{d}")


def _same_bits(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_multi_append_then_attention(gpu_lib, oracle_mod, case):
    b, h, g, n, lens, dtype, d = _unpack(case)
    pb = MultiProblem(b, h, g, n, lens, seed=1200 + h + g + n + d, dtype=dtype, d=d)
    q, kn, vn = pb.draw_step()
    api.kv_append_multi(pb.kc, pb.vc, to_dev(kn), to_dev(vn), pb.lens, int(max(lens)))
    out = torch.empty(b, n, h, d, dtype=pb.tdt, device="cuda")
    api.decode_attention_multi(out, to_dev(q), pb.kc, pb.vc, pb.lens, int(max(lens)) + n, pb.scale, pb.ws)
    torch.cuda.synchronize()
    oracle_mod.kv_append_multi(pb.kc_h, pb.vc_h, kn, vn, pb.lens_h)
    assert np.array_equal(pb.lens.cpu().numpy(), pb.lens_h)
    assert _same_bits(to_host_bits(pb.kc), pb.kc_h) and _same_bits(to_host_bits(pb.vc), pb.vc_h)
    want = oracle_mod.decode_attention_multi(q, pb.kc_h, pb.vc_h, pb.lens_h, pb.scale)
    assert_parity(out, want, dtype, f"multi-token {case}")


@pytest.mark.parametrize("case", CASES[:5] + CASES[7:], ids=_id)
def test_multi_step_loop(gpu_lib, oracle_mod, case):
    b, h, g, n, lens, dtype, d = _unpack(case)
    steps = 3
    pb = MultiProblem(b, h, g, n, lens, seed=1300 + h + g + n + d, steps=steps, dtype=dtype, d=d)
    for step in range(steps):
        q, kn, vn = pb.draw_step()
        max_len = int(pb.lens_h.max())
        out = torch.empty(b, n, h, d, dtype=pb.tdt, device="cuda")
        api.decode_step_multi(out, to_dev(q), to_dev(kn), to_dev(vn), pb.kc, pb.vc, pb.lens, max_len, pb.scale, pb.ws)
        torch.cuda.synchronize()
        oracle_mod.kv_append_multi(pb.kc_h, pb.vc_h, kn, vn, pb.lens_h)
        want = oracle_mod.decode_attention_multi(q, pb.kc_h, pb.vc_h, pb.lens_h, pb.scale)
        assert_parity(out, want, dtype, f"multi step {step} {case}")
        assert np.array_equal(pb.lens.cpu().numpy(), pb.lens_h)
        assert _same_bits(to_host_bits(pb.kc), pb.kc_h)


def test_one_token_multi_equals_the_one_token_call(gpu_lib):
    b, h, g = 3, 64, 8
    pb = MultiProblem(b, h, g, 1, [100, 2000, 4097], seed=1400)
    q, _, _ = pb.draw_step()
    max_len = int(pb.lens_h.max())
    out = torch.empty(b, 1, h, 128, dtype=torch.bfloat16, device="cuda")
    api.decode_attention_multi(out, to_dev(q), pb.kc, pb.vc, pb.lens, max_len, pb.scale, pb.ws)
    ref = torch.empty(b, h, 128, dtype=torch.bfloat16, device="cuda")
    ws = api.make_workspace(b, h, g, 128, 128, max_len, torch.bfloat16, "cuda")
    api.decode_attention(ref, to_dev(np.ascontiguousarray(q[:, 0])), pb.kc, pb.vc, pb.lens, max_len, pb.scale, ws,
                         path=api.PATH_MATRIX)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0].view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("b,h,g,n,lens", [(3, 64, 8, 4, [1, 29, 511]), (4, 28, 4, 3, [0, 62, 63, 200]),
                                           (3, 64, 8, 2, [0, 31, 300]), (2, 64, 8, 8, [5, 700]),
                                           (2, 24, 4, 8, [3, 260])])
def test_multi_step_equals_append_then_attention(gpu_lib, b, h, g, n, lens):
    # the one-launch step (new rows stored by the tiles that hold them) and the
    # two calls give the same bits: the same tile states folded in the same order
    print(f"multi-token step against the two calls: h={h} g={g} n={n} lens={lens}", flush=True)
    one = MultiProblem(b, h, g, n, lens, seed=1450 + n)
    two = MultiProblem(b, h, g, n, lens, seed=1450 + n)
    q, kn, vn = one.draw_step()
    max_len = int(one.lens_h.max())
    out1 = torch.empty(b, n, h, 128, dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out1)
    api.decode_step_multi(out1, to_dev(q), to_dev(kn), to_dev(vn), one.kc, one.vc, one.lens, max_len, one.scale,
                          one.ws)
    api.kv_append_multi(two.kc, two.vc, to_dev(kn), to_dev(vn), two.lens, max_len)
    api.decode_attention_multi(out2, to_dev(q), two.kc, two.vc, two.lens, max_len + n, two.scale, two.ws)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(one.lens, two.lens)
    assert torch.equal(one.kc.view(torch.int16), two.kc.view(torch.int16))
    assert torch.equal(one.vc.view(torch.int16), two.vc.view(torch.int16))


def test_multi_rejects(gpu_lib):
    pb = MultiProblem(2, 64, 8, 2, [10, 20], seed=1500)
    q = torch.zeros(2, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(RuntimeError, match="WORKSPACE"):   # a one-token workspace is too small for 2 tokens
        api.decode_attention_multi(out, q, pb.kc, pb.vc, pb.lens, 22, pb.scale,
                                   api.make_workspace(2, 64, 8, 128, 128, 22, torch.bfloat16, "cuda"))
    with pytest.raises(RuntimeError, match="CAPACITY"):
        api.decode_step_multi(out, q, torch.zeros(2, 2, 8, 128, dtype=torch.bfloat16, device="cuda"),
                              torch.zeros(2, 2, 8, 128, dtype=torch.bfloat16, device="cuda"), pb.kc, pb.vc, pb.lens,
                              pb.cap - 1, pb.scale, pb.ws)
    assert np.array_equal(pb.lens.cpu().numpy(), pb.lens_h)  # nothing was enqueued


@pytest.mark.parametrize("n", [4, 8])
def test_multi_llama3_70b_shape(gpu_lib, oracle_mod, n):
    # the Llama-3-70B-shaped batch with 4 or 8 speculative tokens per sequence (32 or 64 virtual heads
    # per group; with 8, two folding waves of 32 heads merge the split segments inside the launch)
    wl = WORKLOADS["llama3_70b_gqa_bf16"]
    print(f"multi-token step: Llama-3-70B shape, n={n}", flush=True)
    batch = inputs.Batch(seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=wl.lens, dtype="bf16",
                         poison=True)
    rng = np.random.default_rng(7)
    q, kn, vn = (_draw(rng, (wl.b, n, x, 128)) for x in (wl.h, wl.g, wl.g))
    kc, vc = to_dev(batch.k_cache), to_dev(batch.v_cache)
    lens = torch.from_numpy(batch.lens.copy()).cuda()
    ws = api.make_multi_workspace(wl.b, n, wl.h, wl.g, 128, 128, torch.bfloat16, "cuda")
    out = torch.empty(wl.b, n, wl.h, 128, dtype=torch.bfloat16, device="cuda")
    api.decode_step_multi(out, to_dev(q), to_dev(kn), to_dev(vn), kc, vc, lens, int(batch.lens.max()), wl.scale, ws)
    torch.cuda.synchronize()
    kc_h, vc_h, lens_h = batch.k_cache, batch.v_cache, batch.lens.copy()
    oracle_mod.kv_append_multi(kc_h, vc_h, kn, vn, lens_h)
    want = oracle_mod.decode_attention_multi(q, kc_h, vc_h, lens_h, wl.scale, threads=16)
    assert_parity(out, want, "bf16", "multi-token Llama-3-70B shape")
