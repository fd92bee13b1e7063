"""GPU parity of the KV-head mean-fold (gqa_fold_kv_heads) against the oracle.

Both sides sum the F heads of a group in head order in double precision and
round the mean once to the element type, so the comparison is bit for bit.
Rows at or beyond each sequence's length hold a sentinel that must survive.
The lesson's lab rule is checked on the GPU too: folding with g_dst = g_src
leaves the attention output exactly MHA's, and fewer KV heads change it.
"""
import numpy as np
import pytest
import torch

from gpu_util import to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from gqa_kv_cache_decode_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7E01  # a NaN pattern no fold produces
SENTINEL_F32 = np.float32(-7.25)


def _draw(seed, shape, dtype, spread=False):
    rng = np.random.default_rng(seed)
    vals = rng.standard_normal(shape)
    if spread:  # magnitudes over 12 decades: sums that fp32 could not hold exactly
        vals = vals * 10.0 ** rng.integers(-6, 6, shape)
    vals = vals.astype(np.float32)
    return inputs.f32_to_bf16_bits(vals) if dtype == "bf16" else vals


def _sentinel_like(shape, dtype):
    if dtype == "bf16":
        return np.full(shape, SENTINEL_BF16, dtype=np.uint16)
    return np.full(shape, SENTINEL_F32, dtype=np.float32)


def _run(oracle_mod, src, g_dst, lens, cap_dst, dtype, max_rows=None):
    b, g_src, cap_src, d = src.shape
    want = oracle_mod.fold_heads(src, g_dst, lens, out=_sentinel_like((b, g_dst, cap_dst, d), dtype),
                                 max_rows=max_rows)
    dst = to_dev(_sentinel_like((b, g_dst, cap_dst, d), dtype))
    lens_dev = torch.from_numpy(lens).cuda() if lens is not None else None
    rows = max_rows if max_rows is not None else (int(lens.max()) if lens is not None else min(cap_src, cap_dst))
    api.fold_kv_heads(dst, to_dev(src), lens_dev, rows)
    torch.cuda.synchronize()
    got = to_host_bits(dst)
    return got, want


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("g_src,g_dst,d", [(4, 2, 128), (6, 2, 16), (5, 1, 64), (32, 8, 128), (32, 1, 8),
                                           (8, 8, 128), (64, 8, 256), (12, 3, 40)])
def test_fold_parity_ragged(gpu_lib, oracle_mod, dtype, g_src, g_dst, d):
    b, cap = 5, 300
    lens = np.array([0, 1, 255, 256, 300], dtype=np.int32)  # empty, one row, around a 2048-element chunk
    src = _draw(600 + g_src + g_dst + d, (b, g_src, cap, d), dtype, spread=True)
    got, want = _run(oracle_mod, src, g_dst, lens, cap + 7, dtype)
    assert np.array_equal(got.view(np.uint32 if dtype == "f32" else np.uint16),
                          want.view(np.uint32 if dtype == "f32" else np.uint16))


def test_fold_without_lengths_folds_a_projection(gpu_lib, oracle_mod):
    # W_k [g*d_k][d_model] viewed as b = 1, g heads of d_k rows of width d_model
    g, d_k, d_model = 8, 128, 1024
    w = inputs.draw_weight(31, 1, g * d_k, d_model, "bf16")
    got, want = _run(oracle_mod, w.reshape(1, g, d_k, d_model), 2, None, d_k, "bf16", max_rows=d_k)
    assert np.array_equal(got, want)


def test_fold_rounds_once_and_handles_inf_and_nan(gpu_lib, oracle_mod):
    # heads 4, 2^-6, 2^-28, 0 average to 1 + 2^-8 + 2^-30 (just above a bf16 tie): 0x3F81;
    # a group holding +inf gives inf, one holding +inf and -inf gives the canonical NaN
    cols = [
        [4.0, 2.0 ** -6, 2.0 ** -28, 0.0],
        [np.inf, 1.0, 2.0, 3.0],
        [np.inf, -np.inf, 0.0, 0.0],
        [3.0e38, 3.0e38, 3.0e38, 3.0e38],   # the sum passes fp32's range, the mean does not
        [1e-40, 0.0, 0.0, 0.0],             # subnormal
        [-2.0 ** -133, 0.0, 0.0, 0.0],      # rounds to -0
    ]
    vals = np.zeros((1, 4, 1, 8), dtype=np.float32)
    for c, col in enumerate(cols):
        vals[0, :, 0, c] = col
    src = inputs.f32_to_bf16_bits(vals)
    got, want = _run(oracle_mod, src, 1, None, 1, "bf16", max_rows=1)
    assert np.array_equal(got, want)
    assert got[0, 0, 0, 0] == 0x3F81 and got[0, 0, 0, 1] == 0x7F80 and got[0, 0, 0, 2] == 0x7FC0
    assert got[0, 0, 0, 5] == 0x8000


def test_fold_rejects(gpu_lib):
    src = torch.zeros(1, 6, 4, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="g_src=6 is not a multiple"):
        api.fold_kv_heads(torch.zeros(1, 4, 4, 8, dtype=torch.bfloat16, device="cuda"), src)
    with pytest.raises(RuntimeError, match="exceeds"):
        api.fold_kv_heads(torch.zeros(1, 3, 4, 8, dtype=torch.bfloat16, device="cuda"), src, max_rows=5)
    with pytest.raises(RuntimeError, match="overlap"):
        big = torch.zeros(1, 6, 4, 8, dtype=torch.bfloat16, device="cuda")
        api.fold_kv_heads(big[:, :3], big)  # in place is not allowed


def test_fold_long_mha_cache_sampled_sequences(gpu_lib, oracle_mod):
    # the long MHA workload's cache (b=4, g=32, L=32769, d=128, bf16) folded to g=8;
    # sequences 0 and 3 are compared whole against the oracle
    wl = WORKLOADS["mha_long_bf16_g32"]
    L = wl.lens + 1
    batch = inputs.Batch(seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=[L] * wl.b, dtype="bf16",
                         poison=True)
    lens = batch.lens.copy()
    print(f"fold: {wl.name} K cache, {wl.b}x{wl.g}x{L}x{wl.d} -> g=8", flush=True)
    dst = torch.full((wl.b, 8, wl.cap, wl.d), 0.0, dtype=torch.bfloat16, device="cuda")
    api.fold_kv_heads(dst, to_dev(batch.k_cache), torch.from_numpy(lens).cuda(), int(lens.max()))
    torch.cuda.synchronize()
    got = to_host_bits(dst)
    for s in (0, 3):
        want = oracle_mod.fold_heads(np.ascontiguousarray(batch.k_cache[s:s + 1]), 8, lens[s:s + 1])
        assert np.array_equal(got[s:s + 1, :, :L], want[:, :, :L]), s


def test_fold_lab_rule_on_gpu(gpu_lib):
    # same weights (cache, queries): g_dst = g_src keeps MHA's output bit for bit, fewer KV
    # heads change it, and the grouped decode over the folded cache reads g/h of the bytes
    b, h, d, L, cap = 4, 32, 128, 1500, 1600
    batch = inputs.Batch(seed=77, b=b, h=h, g=h, d=d, cap=cap, lens=[L] * b, dtype="bf16", poison=False)
    kc, vc = to_dev(batch.k_cache), to_dev(batch.v_cache)
    lens = torch.from_numpy(batch.lens.copy()).cuda()
    q = to_dev(batch.q(0))
    scale = float(np.float32(1.0 / np.sqrt(d)))

    def attend(k, v, g):
        out = torch.empty(b, h, d, dtype=torch.bfloat16, device="cuda")
        ws = api.make_workspace(b, h, g, d, d, L, torch.bfloat16, "cuda")
        api.decode_attention(out, q, k, v, lens, L, scale, ws)
        return out

    mha = attend(kc, vc, h)
    deltas = {}
    for g in (32, 8, 1):
        kf = torch.empty(b, g, cap, d, dtype=torch.bfloat16, device="cuda")
        vf = torch.empty_like(kf)
        api.fold_kv_heads(kf, kc, lens, L)
        api.fold_kv_heads(vf, vc, lens, L)
        out = attend(kf, vf, g)
        torch.cuda.synchronize()
        diff = (out.float() - mha.float()).norm() / mha.float().norm()
        deltas[g] = float(diff)
        if g == h:
            assert torch.equal(out.view(torch.int16), mha.view(torch.int16))
        else:
            assert deltas[g] > 0.1
    print("output delta vs MHA:", deltas, flush=True)
