"""GPU parity of the paged-cache entry points (gqa_kv_append_paged,
gqa_decode_attention_paged, gqa_decode_step_paged).

Every case lays one seeded contiguous cache out as a pool with a shuffled
block table (spare blocks and rows past the lengths NaN-poisoned, table
entries past a sequence's last block -1) and checks
* the attention against the fp64 oracle over the cache the pool stands for,
  to the decode parity bar;
* that the paged call returns exactly (bit for bit) what the contiguous call
  returns on the same data: same kernels, same schedule, same arithmetic;
* for appends and fused steps, that the new rows land in the right block
  rows, bit for bit, that nothing else in the pool changed, and that the
  lengths grew by one.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from gqa_kv_cache_decode_amd.workloads import WORKLOADS
from paged_util import make_paged

pytestmark = pytest.mark.gpu


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality (NaN poison included)."""
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


CASES = [
    # dtype, b, h, g, d, lens, block_size   (path chosen by the library)
    ("bf16", 4, 64, 8, 128, [0, 31, 32, 300], 32),        # matrix, G = 8
    ("bf16", 3, 28, 4, 128, [1, 200, 511], 64),           # matrix, G = 7
    ("bf16", 2, 32, 1, 128, [700, 1500], 256),            # matrix, G = 32, merged by a second launch
    ("bf16", 2, 64, 1, 128, [300, 77], 64),               # matrix, G = 64: four head blocks
    ("bf16", 3, 8, 4, 128, [5, 64, 190], 32),             # vector, G = 2
    ("bf16", 2, 16, 16, 64, [33, 129], 128),              # vector, MHA
    ("f32", 2, 4, 2, 16, [37, 64], 32),                   # vector, fp32
    ("f32", 3, 12, 3, 256, [0, 95, 96], 32),              # vector, fp32, d = 256
]


class PagedProblem:
    def __init__(self, dtype, b, h, g, d, lens, block_size, seed, cap=None, room=1):
        self.dtype, self.b, self.h, self.g, self.d, self.bs = dtype, b, h, g, d, block_size
        cap = cap or (max(lens) + 8 + block_size - 1) // block_size * block_size
        self.batch = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
        self.cap = cap
        rng = np.random.default_rng(seed)
        self.kp, self.table = make_paged(self.batch.k_cache, self.batch.lens, block_size, rng, room=room)
        self.vp, _ = make_paged(self.batch.v_cache, self.batch.lens, block_size, np.random.default_rng(seed),
                                room=room)
        self.scale = float(np.float32(1.0 / np.sqrt(d)))
        self.tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def device(self):
        return (to_dev(self.kp), to_dev(self.vp), torch.from_numpy(self.table).cuda(),
                torch.from_numpy(self.batch.lens.copy()).cuda())

    def workspace(self, max_len):
        return api.make_workspace(self.b, self.h, self.g, self.d, self.d, max_len, self.tdt, "cuda")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-h{c[2]}g{c[3]}d{c[4]}-B{c[6]}")
def test_paged_attention_parity_and_identity(gpu_lib, oracle_mod, case):
    dtype, b, h, g, d, lens, bs = case
    pb = PagedProblem(dtype, b, h, g, d, lens, bs, seed=700 + h + bs)
    kp, vp, table, lens_d = pb.device()
    q = to_dev(pb.batch.q(0))
    max_len = int(max(lens))
    out = torch.empty(b, h, d, dtype=pb.tdt, device="cuda")
    api.decode_attention_paged(out, q, kp, vp, lens_d, table, max_len, pb.scale, pb.workspace(max_len))
    # the contiguous call on the cache the pool stands for
    ref_out = torch.empty_like(out)
    api.decode_attention(ref_out, q, to_dev(pb.batch.k_cache), to_dev(pb.batch.v_cache), lens_d, max_len, pb.scale,
                         pb.workspace(max_len))
    torch.cuda.synchronize()
    want = oracle_mod.decode_attention_paged(pb.batch.q(0), pb.kp, pb.vp, pb.batch.lens, pb.table, pb.scale)
    assert_parity(out, want, dtype, f"paged attention {case}")
    assert same_bits(to_host_bits(out), to_host_bits(ref_out))
    # nothing was written to the pool
    assert same_bits(to_host_bits(kp), pb.kp) and same_bits(to_host_bits(vp), pb.vp)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-h{c[2]}g{c[3]}d{c[4]}-B{c[6]}")
def test_paged_append_bitwise(gpu_lib, oracle_mod, case):
    dtype, b, h, g, d, lens, bs = case
    pb = PagedProblem(dtype, b, h, g, d, lens, bs, seed=800 + h + bs)
    kp, vp, table, lens_d = pb.device()
    kn, vn = pb.batch.new_kv(0)
    api.kv_append_paged(kp, vp, to_dev(kn), to_dev(vn), lens_d, table, int(max(lens)))
    torch.cuda.synchronize()
    kp_h, vp_h, lens_h = pb.kp.copy(), pb.vp.copy(), pb.batch.lens.copy()
    oracle_mod.kv_append_paged(kp_h, vp_h, kn, vn, lens_h, pb.table)
    assert np.array_equal(lens_d.cpu().numpy(), lens_h)
    assert same_bits(to_host_bits(kp), kp_h) and same_bits(to_host_bits(vp), vp_h)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-h{c[2]}g{c[3]}d{c[4]}-B{c[6]}")
def test_paged_step_loop(gpu_lib, oracle_mod, case):
    # several fused steps in a row, crossing block boundaries; each step against the oracle
    # (append, then attention over the grown cache) and against the contiguous fused step
    dtype, b, h, g, d, lens, bs = case
    steps = 4
    pb = PagedProblem(dtype, b, h, g, d, lens, bs, seed=900 + h + bs, room=steps)
    kp, vp, table, lens_d = pb.device()
    kc, vc = to_dev(pb.batch.k_cache), to_dev(pb.batch.v_cache)
    lens_c = lens_d.clone()
    kp_h, vp_h, lens_h = pb.kp.copy(), pb.vp.copy(), pb.batch.lens.copy()
    ws = pb.workspace(int(max(lens)) + steps + 1)
    ws_c = pb.workspace(int(max(lens)) + steps + 1)
    for step in range(steps):
        q = pb.batch.q(step)
        kn, vn = pb.batch.new_kv(step)
        max_len = int(lens_h.max())
        out = torch.empty(b, h, d, dtype=pb.tdt, device="cuda")
        api.decode_step_paged(out, to_dev(q), to_dev(kn), to_dev(vn), kp, vp, lens_d, table, max_len, pb.scale, ws)
        out_c = torch.empty_like(out)
        api.decode_step(out_c, to_dev(q), to_dev(kn), to_dev(vn), kc, vc, lens_c, max_len, pb.scale, ws_c)
        torch.cuda.synchronize()
        oracle_mod.kv_append_paged(kp_h, vp_h, kn, vn, lens_h, pb.table)
        want = oracle_mod.decode_attention_paged(q, kp_h, vp_h, lens_h, pb.table, pb.scale)
        assert_parity(out, want, dtype, f"paged step {step} {case}")
        assert same_bits(to_host_bits(out), to_host_bits(out_c)), f"step {step}"
        assert np.array_equal(lens_d.cpu().numpy(), lens_h)
        assert same_bits(to_host_bits(kp), kp_h) and same_bits(to_host_bits(vp), vp_h)


def test_paged_llama3_70b_shape_matches_contiguous(gpu_lib):
    # the Llama-3-70B-shaped batch (b=16, h=64, g=8, d=128, lengths U[1024, 8192]) in blocks
    # of 256 positions: the fused paged step equals the contiguous one bit for bit, and the
    # pool holds exactly the contiguous cache's rows afterwards
    wl = WORKLOADS["llama3_70b_gqa_bf16"]
    print("paged step: Llama-3-70B shape, blocks of 256", flush=True)
    batch = inputs.Batch(seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=wl.lens, dtype="bf16",
                         poison=True)
    rng = np.random.default_rng(5)
    kp, table = make_paged(batch.k_cache, batch.lens, 256, rng)
    vp, _ = make_paged(batch.v_cache, batch.lens, 256, np.random.default_rng(5))
    kp_d, vp_d, table_d = to_dev(kp), to_dev(vp), torch.from_numpy(table).cuda()
    kc, vc = to_dev(batch.k_cache), to_dev(batch.v_cache)
    lens_p = torch.from_numpy(batch.lens.copy()).cuda()
    lens_c = lens_p.clone()
    q = to_dev(batch.q(0))
    kn, vn = (to_dev(a) for a in batch.new_kv(0))
    max_len = int(batch.lens.max())
    ws = api.make_workspace(wl.b, wl.h, wl.g, wl.d, wl.d, max_len + 1, torch.bfloat16, "cuda")
    out = torch.empty(wl.b, wl.h, wl.d, dtype=torch.bfloat16, device="cuda")
    out_c = torch.empty_like(out)
    api.decode_step_paged(out, q, kn, vn, kp_d, vp_d, lens_p, table_d, max_len, wl.scale, ws)
    api.decode_step(out_c, q, kn, vn, kc, vc, lens_c, max_len, wl.scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(lens_p, lens_c)
    lens_h = lens_c.cpu().numpy()
    kp_h, kc_h = to_host_bits(kp_d), to_host_bits(kc)
    for s in (0, 7, 15):
        t = np.arange(lens_h[s])
        assert np.array_equal(kp_h[table[s, t // 256], :, t % 256].transpose(1, 0, 2), kc_h[s, :, :lens_h[s]])
