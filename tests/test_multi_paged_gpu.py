"""GPU parity of multi-token decode over paged caches (gqa_kv_append_multi_paged,
gqa_decode_attention_multi_paged, gqa_decode_step_multi_paged) against the
fp64 oracle.

Each case lays a seeded, NaN-poisoned contiguous cache out as a pool with a
shuffled block table (room for the appended tokens, spare blocks poisoned,
unused entries -1), appends n tokens per sequence (crossing block
boundaries) and checks
* the whole pool after the append, bit for bit, against the oracle's paged
  append (the new rows in their block rows, nothing else changed), and the
  lengths;
* the outputs of every token and head against the oracle's causal attention
  over the cache the pool stands for, to the decode parity bar;
* that they equal, bit for bit, the contiguous multi-token call on that cache
  (same kernels, same schedule, same arithmetic);
on the matrix kernels (one, two and four 16-row head blocks, the split merge
by a second launch) and the vector path (fp32, other head dims, two or more
than 64 virtual heads); plus a three-step loop and the host-side rejections.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from paged_util import make_paged

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, b, h, g, d, n, pre-append lengths, block size
    ("bf16", 3, 64, 8, 128, 4, [0, 30, 300], 32),     # 32 virtual heads: two MFMA blocks
    ("bf16", 3, 64, 8, 128, 2, [1, 29, 511], 256),    # 16: one block, eight waves
    ("bf16", 2, 64, 8, 128, 8, [5, 700], 64),         # 64: four blocks
    ("bf16", 2, 32, 1, 128, 2, [900, 3000], 128),     # MQA: split merge by a second launch
    ("bf16", 3, 8, 8, 128, 2, [3, 33, 97], 32),       # 2 virtual heads: vector path
    ("f32", 3, 8, 4, 16, 3, [0, 31, 100], 32),        # fp32, d = 16
    ("bf16", 2, 16, 4, 64, 4, [10, 200], 64),         # bf16, d = 64
    ("bf16", 2, 72, 8, 128, 8, [64, 300], 32),        # 72 virtual heads: vector path
]


def _id(c):
    return f"{c[0]}-h{c[2]}g{c[3]}d{c[4]}-n{c[5]}-B{c[7]}"


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


class Problem:
    def __init__(self, dtype, b, h, g, d, n, lens, bs, seed, steps=1):
        self.dtype, self.b, self.h, self.g, self.d, self.n, self.bs = dtype, b, h, g, d, n, bs
        self.tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        cap = (max(lens) + n * steps + 8 + bs - 1) // bs * bs
        self.cap = cap
        bt = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
        self.rng = np.random.default_rng(seed)
        self.kp_h, self.table_h = make_paged(bt.k_cache, bt.lens, bs, np.random.default_rng(seed + 1),
                                             room=n * steps)
        self.vp_h, _ = make_paged(bt.v_cache, bt.lens, bs, np.random.default_rng(seed + 1), room=n * steps)
        self.lens_h = bt.lens.copy()
        self.kp, self.vp = to_dev(self.kp_h), to_dev(self.vp_h)
        self.table = torch.from_numpy(self.table_h).cuda()
        self.lens = torch.from_numpy(self.lens_h.copy()).cuda()
        self.scale = float(np.float32(1.0 / np.sqrt(d)))
        self.ws = api.make_multi_workspace(b, n, h, g, d, d, self.tdt, "cuda")

    def draw(self, *shape):
        x = self.rng.standard_normal(shape).astype(np.float32)
        return inputs.f32_to_bf16_bits(x) if self.dtype == "bf16" else x

    def draw_step(self):
        b, n, h, g, d = self.b, self.n, self.h, self.g, self.d
        return self.draw(b, n, h, d), self.draw(b, n, g, d), self.draw(b, n, g, d)

    def check_state(self, what):
        assert np.array_equal(self.lens.cpu().numpy(), self.lens_h), what
        assert np.array_equal(_bits(to_host_bits(self.kp)), _bits(self.kp_h)), what
        assert np.array_equal(_bits(to_host_bits(self.vp)), _bits(self.vp_h)), what

    def contiguous_out(self, oracle_mod, q, max_len):
        """The contiguous multi-token call on the cache the (oracle-updated) pool stands for."""
        cap = self.table_h.shape[1] * self.bs
        kc = oracle_mod.gather_paged(self.kp_h, self.table_h, self.lens_h, self.bs, cap)
        vc = oracle_mod.gather_paged(self.vp_h, self.table_h, self.lens_h, self.bs, cap)
        out = torch.empty(self.b, self.n, self.h, self.d, dtype=self.tdt, device="cuda")
        api.decode_attention_multi(out, to_dev(q), to_dev(kc), to_dev(vc), self.lens, max_len, self.scale,
                                   api.make_multi_workspace(self.b, self.n, self.h, self.g, self.d, self.d, self.tdt,
                                                            "cuda"))
        return out


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_multi_paged_append_then_attention(gpu_lib, oracle_mod, case):
    dtype, b, h, g, d, n, lens, bs = case
    print(f"multi-token paged: {case}", flush=True)
    pb = Problem(dtype, b, h, g, d, n, lens, bs, seed=1600 + h + g + n + bs)
    q, kn, vn = pb.draw_step()
    api.kv_append_multi_paged(pb.kp, pb.vp, to_dev(kn), to_dev(vn), pb.lens, pb.table, int(max(lens)))
    out = torch.empty(b, n, h, d, dtype=pb.tdt, device="cuda")
    max_len = int(max(lens)) + n
    api.decode_attention_multi_paged(out, to_dev(q), pb.kp, pb.vp, pb.lens, pb.table, max_len, pb.scale, pb.ws)
    torch.cuda.synchronize()
    oracle_mod.kv_append_multi_paged(pb.kp_h, pb.vp_h, kn, vn, pb.lens_h, pb.table_h)
    pb.check_state(f"append {case}")
    want = oracle_mod.decode_attention_multi_paged(q, pb.kp_h, pb.vp_h, pb.lens_h, pb.table_h, pb.scale)
    assert_parity(out, want, dtype, f"multi-token paged {case}")
    ref = pb.contiguous_out(oracle_mod, q, max_len)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if dtype == "bf16" else torch.int32),
                       ref.view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[5], CASES[7]], ids=_id)
def test_multi_paged_step_loop(gpu_lib, oracle_mod, case):
    dtype, b, h, g, d, n, lens, bs = case
    steps = 3
    pb = Problem(dtype, b, h, g, d, n, lens, bs, seed=1700 + h + g + n + bs, steps=steps)
    for step in range(steps):
        print(f"multi-token paged step {step}: {case}", flush=True)
        q, kn, vn = pb.draw_step()
        max_len = int(pb.lens_h.max())
        out = torch.empty(b, n, h, d, dtype=pb.tdt, device="cuda")
        api.decode_step_multi_paged(out, to_dev(q), to_dev(kn), to_dev(vn), pb.kp, pb.vp, pb.lens, pb.table, max_len,
                                    pb.scale, pb.ws)
        torch.cuda.synchronize()
        oracle_mod.kv_append_multi_paged(pb.kp_h, pb.vp_h, kn, vn, pb.lens_h, pb.table_h)
        pb.check_state(f"step {step} {case}")
        want = oracle_mod.decode_attention_multi_paged(q, pb.kp_h, pb.vp_h, pb.lens_h, pb.table_h, pb.scale)
        assert_parity(out, want, dtype, f"multi-token paged step {step} {case}")


def test_multi_paged_rejects(gpu_lib):
    pb = Problem("bf16", 2, 64, 8, 128, 2, [10, 20], 32, seed=1800)
    q = torch.zeros(2, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(2, 2, 8, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    room = pb.table_h.shape[1] * pb.bs
    with pytest.raises(RuntimeError, match="CAPACITY"):      # no room for 2 more tokens
        api.decode_step_multi_paged(out, q, kn, kn.clone(), pb.kp, pb.vp, pb.lens, pb.table, room - 1, pb.scale,
                                    pb.ws)
    with pytest.raises(RuntimeError, match="CAPACITY"):
        api.kv_append_multi_paged(pb.kp, pb.vp, kn, kn.clone(), pb.lens, pb.table, room - 1)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):   # block size not a power of two >= 32
        api.decode_attention_multi_paged(out, q, pb.kp[:, :, :16].contiguous(), pb.vp[:, :, :16].contiguous(),
                                         pb.lens, pb.table, 22, pb.scale, pb.ws)
    torch.cuda.synchronize()
    pb.check_state("nothing was enqueued")
