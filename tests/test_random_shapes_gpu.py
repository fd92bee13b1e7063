"""Parity over a fixed set of randomly drawn shapes (seeded; the same cases
every run): batch, head counts, head dim, element type, ragged lengths with
empty sequences, kernel path, merge mode, grid size and call form (two calls
or the fused step) all vary together, so that combinations the hand-picked
cases miss are held to the same bar against the fp64 oracle; a second set
draws the stream kernel's shapes with their split segments merged by the
parts at the end of the launch (GQA_MERGE_SPREAD).
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_counters_zero, assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        d = int(rng.choice([16, 32, 64, 128, 128, 128, 256]))
        g = int(rng.choice([1, 1, 2, 3, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 32, 48, 64]))
        b = int(rng.integers(1, 24))
        lens = rng.integers(0, 700, b)
        lens[rng.random(b) < 0.15] = 0
        matrix_ok = dtype == "bf16" and d == 128 and G <= 64
        path = int(rng.choice([api.PATH_AUTO, api.PATH_VECTOR] + ([api.PATH_MATRIX] if matrix_ok else [])))
        merge = int(rng.choice([0, api.MERGE_INLINE, api.MERGE_KERNEL]))
        wgs = int(rng.choice([0, 0, 1, 7, 64, 300, 2048]))
        fused = bool(rng.random() < 0.5)
        out.append((k, dtype, b, g * G, g, d, [int(x) for x in lens], path | merge, wgs, fused))
    return out


def _spread_cases(n=24, seed=20261203):
    # shapes the stream kernel runs (bf16, d = 128, 3-64 heads per KV head, b <= 64), split
    # segments merged by their parts at the end of the launch (GQA_MERGE_SPREAD)
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        g = int(rng.choice([1, 1, 2, 3, 4, 8]))
        G = int(rng.choice([3, 4, 5, 7, 8, 12, 16, 17, 24, 32, 33, 48, 64]))
        b = int(rng.integers(1, 65))
        lens = rng.integers(0, 900, b)
        lens[rng.random(b) < 0.15] = 0
        path = int(rng.choice([api.PATH_AUTO, api.PATH_MATRIX])) | api.MERGE_SPREAD
        wgs = int(rng.choice([0, 0, 1, 7, 64, 300, 2048]))
        fused = bool(rng.random() < 0.5)
        out.append((100 + k, "bf16", b, g * G, g, 128, [int(x) for x in lens], path, wgs, fused))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_shape(gpu_lib, oracle_mod, case):
    _run_case(oracle_mod, case)


@pytest.mark.parametrize("case", _spread_cases(), ids=lambda c: f"spread{c[0]}")
def test_random_shape_spread_merge(gpu_lib, oracle_mod, case):
    _run_case(oracle_mod, case)


def _run_case(oracle_mod, case):
    k, dtype, b, h, g, d, lens, path, wgs, fused = case
    cap = max(lens) + 3
    bt = inputs.Batch(seed=3000 + k, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = float(np.float32(1.0 / np.sqrt(d)))
    kc, vc = to_dev(bt.k_cache), to_dev(bt.v_cache)
    lens_d = torch.from_numpy(bt.lens.copy()).cuda()
    q = bt.q(0)
    kn, vn = bt.new_kv(0)
    max_len = int(bt.lens.max())
    ws = api.make_workspace(b, h, g, d, d, max_len + 1, tdt, "cuda")
    out = torch.empty(b, h, d, dtype=tdt, device="cuda")
    if fused:
        api.decode_step(out, to_dev(q), to_dev(kn), to_dev(vn), kc, vc, lens_d, max_len, scale, ws, path=path,
                        workgroups=wgs)
    else:
        api.kv_append(kc, vc, to_dev(kn), to_dev(vn), lens_d, max_len)
        api.decode_attention(out, to_dev(q), kc, vc, lens_d, max_len + 1, scale, ws, path=path, workgroups=wgs)
    torch.cuda.synchronize()
    kh, vh, lh = bt.k_cache.copy(), bt.v_cache.copy(), bt.lens.copy()
    oracle_mod.kv_append(kh, vh, kn, vn, lh)
    assert np.array_equal(lens_d.cpu().numpy(), lh)
    assert np.array_equal(to_host_bits(kc).view(np.uint8), kh.view(np.uint8))
    assert np.array_equal(to_host_bits(vc).view(np.uint8), vh.view(np.uint8))
    assert_parity(out, oracle_mod.decode_attention(q, kh, vh, lh, scale), dtype, f"case {case}")
    assert_counters_zero(ws, b, h)
