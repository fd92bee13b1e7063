"""GPU parity of the projections (gqa_linear) and of the whole-layer decode step
(gqa_decode_layer) against the fp64 oracle.

The projection outputs are O(1) (x ~ N(0, 1), weights ~ N(0, 1/n_in)) and are
held to the decode parity bar for bf16. The layer is checked end to end
(output projection), at every intermediate (q, k_new, v_new, attention
output), and on the cache: the appended rows are exactly the projections the
GPU produced, and the lengths grew by one.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_counters_zero, assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from gqa_kv_cache_decode_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows", [1, 7, 16, 17, 33, 64])
@pytest.mark.parametrize("n_in,n_out", [(8, 1), (40, 17), (128, 100), (1000, 48), (8192, 1024)])
def test_linear_parity(gpu_lib, oracle_mod, rows, n_in, n_out):
    x = inputs.normals(11, (rows, n_in), rows * n_in, "bf16").reshape(rows, n_in)
    w = inputs.draw_weight(12 + n_out, 0, n_out, n_in, "bf16")
    y = torch.empty(rows, n_out, dtype=torch.bfloat16, device="cuda")
    api.linear(y, to_dev(x), api.PackedWeight(to_dev(w)))
    torch.cuda.synchronize()
    assert_parity(y, oracle_mod.linear(x, w), "bf16", f"rows={rows} n_in={n_in} n_out={n_out}")


@pytest.mark.parametrize("n_out,n_in", [(1, 8), (17, 40), (48, 1000), (64, 96)])
def test_pack_weight_layout(gpu_lib, n_out, n_in):
    # tile (block, s): lane l = 16q + n holds row 16*block + n, columns 32s + 8q .. +7; zero padding
    w = inputs.draw_weight(15, 0, n_out, n_in, "bf16")
    packed = api.PackedWeight(to_dev(w))
    torch.cuda.synchronize()
    got = packed.data.cpu().numpy().view(np.uint16)
    nb, ns = (n_out + 15) // 16, (n_in + 31) // 32
    padded = np.zeros((nb * 16, ns * 32), dtype=np.uint16)
    padded[:n_out, :n_in] = w
    want = padded.reshape(nb, 16, ns, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert got.size == want.size and np.array_equal(got, want)


def test_linear_is_deterministic(gpu_lib):
    x = to_dev(inputs.normals(13, (1,), 16 * 4096, "bf16").reshape(16, 4096))
    w = api.PackedWeight(to_dev(inputs.draw_weight(14, 0, 4096, 4096, "bf16")))
    a = torch.empty(16, 4096, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    api.linear(a, x, w)
    api.linear(b, x, w)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


class LayerProblem:
    def __init__(self, oracle_mod, *, seed, b, h, g, d, d_model, cap, lens):
        self.b, self.h, self.g, self.d, self.d_model = b, h, g, d, d_model
        self.scale = float(np.float32(1.0 / np.sqrt(d)))
        self.batch = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype="bf16", poison=True)
        self.w_q = inputs.draw_weight(seed, 0, h * d, d_model, "bf16")
        self.w_k = inputs.draw_weight(seed, 1, g * d, d_model, "bf16")
        self.w_v = inputs.draw_weight(seed, 2, g * d, d_model, "bf16")
        self.w_o = inputs.draw_weight(seed, 3, d_model, h * d, "bf16")
        self.dev_w = [api.PackedWeight(to_dev(w)) for w in (self.w_q, self.w_k, self.w_v, self.w_o)]
        self.kc, self.vc = to_dev(self.batch.k_cache), to_dev(self.batch.v_cache)
        self.lens_h = self.batch.lens.copy()
        self.lens = torch.from_numpy(self.lens_h.copy()).cuda()
        self.ws = api.make_workspace(b, h, g, d, d, cap, torch.bfloat16, "cuda")
        self.scratch = api.LayerScratch(b, h, g, d, d, torch.bfloat16, "cuda")
        self.oracle = oracle_mod
        self.seed = seed

    def step(self, step):
        x = inputs.draw_x(self.seed, step, self.b, self.d_model, "bf16")
        y = torch.empty(self.b, self.d_model, dtype=torch.bfloat16, device="cuda")
        old = self.lens_h.copy()
        api.decode_layer(y, to_dev(x), *self.dev_w, self.kc, self.vc, self.lens, int(self.lens_h.max()), self.scale,
                         self.ws, self.scratch)
        torch.cuda.synchronize()
        ref, mid = self.oracle.decode_layer(x, self.w_q, self.w_k, self.w_v, self.w_o, self.batch.k_cache,
                                            self.batch.v_cache, self.lens_h, self.scale, self.h)
        return y, ref, mid, old


def _check_layer(pb, step):
    y, ref, mid, old = pb.step(step)
    assert_parity(pb.scratch.q, pb.oracle.linear(
        inputs.draw_x(pb.seed, step, pb.b, pb.d_model, "bf16"), pb.w_q).reshape(pb.b, pb.h, pb.d), "bf16", "q")
    for name, got in (("k_new", pb.scratch.k_new), ("v_new", pb.scratch.v_new), ("attn", pb.scratch.attn)):
        want = inputs.bf16_bits_to_f32(mid[name]).astype(np.float64)
        assert_parity(got, want, "bf16", name)
    assert_parity(y, ref, "bf16", f"layer output, step {step}")
    # the cache holds exactly the rows the GPU projected, at the old lengths
    assert np.array_equal(pb.lens.cpu().numpy(), old + 1)
    kc = to_host_bits(pb.kc)
    vc = to_host_bits(pb.vc)
    kn = to_host_bits(pb.scratch.k_new)
    vn = to_host_bits(pb.scratch.v_new)
    for s in range(pb.b):
        assert np.array_equal(kc[s, :, old[s]], kn[s])
        assert np.array_equal(vc[s, :, old[s]], vn[s])


@pytest.mark.parametrize("h,g,d_model", [(8, 2, 256), (8, 8, 128), (32, 1, 512), (28, 4, 3584 // 7)])
def test_decode_layer_small(gpu_lib, oracle_mod, h, g, d_model):
    pb = LayerProblem(oracle_mod, seed=401 + h + g, b=3, h=h, g=g, d=128, d_model=d_model, cap=80,
                      lens=[0, 5, 70])
    for step in range(2):
        _check_layer(pb, step)


@pytest.mark.parametrize("b", [16, 20, 40])
def test_decode_layer_odd_projection_blocks(gpu_lib, oracle_mod, b):
    # d=16, g=3: the key and value projections have 3 blocks of 16 features each, so
    # from 16 batch rows up (two blocks per workgroup) a workgroup holds a lone last
    # block of each matrix and must not run into the next matrix of the launch
    lens = [(7 * s) % 45 for s in range(b)]
    pb = LayerProblem(oracle_mod, seed=450 + b, b=b, h=6, g=3, d=16, d_model=200, cap=48, lens=lens)
    for step in range(2):
        _check_layer(pb, step)


def test_decode_layer_llama3_70b_shape(gpu_lib, oracle_mod):
    wl = WORKLOADS["llama3_70b_gqa_bf16"]
    print("decode layer: Llama-3-70B shape, d_model=8192", flush=True)
    pb = LayerProblem(oracle_mod, seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, d_model=8192, cap=wl.cap,
                      lens=wl.lens)
    _check_layer(pb, 0)


@pytest.mark.parametrize("b,h,g,d_model,steps", [
    (64, 28, 4, 3584, 2),   # the Qwen2.5-7B shape: 64 batch rows, four 16-row batch blocks
    (33, 16, 2, 1024, 3),   # 33 rows: the last batch block of three holds a single row
    (24, 8, 8, 512, 2),     # 24 rows: two batch blocks; MHA
])
def test_decode_layer_wide_batch(gpu_lib, oracle_mod, b, h, g, d_model, steps):
    # 17-64 batch rows: two to four 16-row batch blocks per projection MFMA, every
    # intermediate and the cache against the oracle over several steps
    print(f"decode layer: b={b} h={h} g={g} d_model={d_model}", flush=True)
    rng = np.random.default_rng(b + h)
    lens = rng.integers(0, 300, b).tolist()
    pb = LayerProblem(oracle_mod, seed=470 + b, b=b, h=h, g=g, d=128, d_model=d_model, cap=max(lens) + steps + 2,
                      lens=lens)
    for step in range(steps):
        _check_layer(pb, step)
    assert_counters_zero(pb.ws, b, h)
