"""GPU check of the allocation-free fused step (gqa_decode_step_static).

It must give exactly what gqa_decode_step gives with a caller workspace on
the same inputs (same kernels, same grid: the outputs, caches and lengths
bit for bit), and meet the parity bar against the fp64 oracle. Two calls in
a row share the library's scratch array; the second has a smaller input, so
it runs on what the first left there.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits, torch_dtype
from gqa_kv_cache_decode_amd import api, inputs

pytestmark = pytest.mark.gpu


class Side:
    """One copy of a problem on the GPU."""

    def __init__(self, batch):
        self.kc, self.vc = to_dev(batch.k_cache), to_dev(batch.v_cache)
        self.lens = torch.from_numpy(batch.lens.copy()).cuda()


def _check(oracle_mod, *, seed, b, h, g, d, cap, lens, dtype):
    batch = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ref_side, static_side = Side(batch), Side(batch)
    q = batch.q(0)
    kn, vn = batch.new_kv(0)
    max_len = int(batch.lens.max())
    tdt = torch_dtype(dtype)
    out_ws = torch.empty(b, h, d, dtype=tdt, device="cuda")
    ws = api.make_workspace(b, h, g, d, d, max_len + 1, tdt, "cuda")
    api.decode_step(out_ws, to_dev(q), to_dev(kn), to_dev(vn), ref_side.kc, ref_side.vc, ref_side.lens, max_len,
                    scale, ws)
    out_st = torch.empty(b, h, d, dtype=tdt, device="cuda")
    api.decode_step_static(out_st, to_dev(q), to_dev(kn), to_dev(vn), static_side.kc, static_side.vc,
                           static_side.lens, max_len, scale)
    torch.cuda.synchronize()
    # the same launch as with a caller workspace: identical bits everywhere
    assert np.array_equal(to_host_bits(out_st).view(np.uint8), to_host_bits(out_ws).view(np.uint8))
    assert torch.equal(static_side.lens, ref_side.lens)
    assert np.array_equal(to_host_bits(static_side.kc).view(np.uint8), to_host_bits(ref_side.kc).view(np.uint8))
    assert np.array_equal(to_host_bits(static_side.vc).view(np.uint8), to_host_bits(ref_side.vc).view(np.uint8))
    # and the oracle's step
    oracle_mod.kv_append(batch.k_cache, batch.v_cache, kn, vn, batch.lens)
    assert np.array_equal(static_side.lens.cpu().numpy(), batch.lens)
    assert np.array_equal(to_host_bits(static_side.kc).view(np.uint8), batch.k_cache.view(np.uint8))
    ref = oracle_mod.decode_attention(q, batch.k_cache, batch.v_cache, batch.lens, scale)
    assert_parity(out_st, ref, dtype, f"static scratch b={b} h={h} g={g} d={d} {dtype}")


def test_static_scratch_step_two_calls(gpu_lib, oracle_mod):
    print("static scratch: Llama-3-70B-shaped call, then a smaller one", flush=True)
    rng = np.random.default_rng(2024)
    # first: the Llama-3-70B shape (one KV group of 8 heads per KV head) with
    # ragged lengths, split over every workgroup
    _check(oracle_mod, seed=2101, b=16, h=64, g=8, d=128, cap=3100,
           lens=rng.integers(1024, 3000, size=16).tolist(), dtype="bf16")
    # second, smaller: fewer sequences and heads, short ragged lengths
    _check(oracle_mod, seed=2102, b=3, h=32, g=4, d=128, cap=400, lens=[5, 130, 390], dtype="bf16")


def test_static_scratch_rejects_oversized_shape(gpu_lib):
    # a shape whose partial slots exceed the 8 MiB array is refused before
    # anything is enqueued (64 heads per KV head, the widest slots)
    b, h, g, d = 64, 4096, 64, 128
    q = torch.zeros(b, h, d, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(b, g, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(b, g, 2, d, dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros(b, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        api.decode_step_static(torch.empty_like(q), q, kn, kn.clone(), kc, kc.clone(), lens, 0, 1.0)
    torch.cuda.synchronize()
    assert int(lens.abs().sum()) == 0
