"""Parity over randomly drawn shapes (seeded; the same cases every run) with
33-64 query heads (or virtual heads, n tokens times h/g) per KV head: the
stream kernel's four-block instances, with two folding waves of 32 heads,
split segments merged inside the launch (up to three parts) or by the second
launch. One-token attention at several grid sizes and both merge modes, the
fused step, the causal multi-token step, over contiguous and paged caches;
outputs against the fp64 oracle at the decode bar, appended rows and lengths
bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_counters_zero, assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from paged_util import make_paged

pytestmark = pytest.mark.gpu

FORMS = ("attention", "step", "multi", "paged_step", "multi_paged")


def _cases(n=30, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        form = FORMS[k % len(FORMS)]
        g = int(rng.choice([1, 2, 4]))
        if form.startswith("multi"):
            ntok = int(rng.choice([2, 3, 4, 8]))
            G = int(rng.integers(-(-33 // ntok), 64 // ntok + 1))  # 33 <= ntok * G <= 64
        else:
            ntok, G = 1, int(rng.integers(33, 65))
        b = int(rng.integers(1, 17))
        lens = rng.integers(1 if form.startswith("multi") else 0, 600, b)
        path = int(rng.choice([api.PATH_AUTO, api.PATH_MATRIX, api.PATH_MATRIX | api.MERGE_INLINE,
                               api.PATH_MATRIX | api.MERGE_KERNEL]))
        wgs = int(rng.choice([0, 0, 1, 5, 64, 256]))
        bs = int(rng.choice([32, 64, 256]))
        out.append((k, form, b, g * G, g, ntok, [int(x) for x in lens], path, wgs, bs))
    return out


def _draw(rng, shape):
    return inputs.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _bits(a):
    return np.ascontiguousarray(a)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-{c[1]}-G{c[3] // c[4]}x{c[5]}")
def test_random_wide_group(gpu_lib, oracle_mod, case):
    k, form, b, h, g, ntok, lens, path, wgs, bs = case
    print(f"wide group case {case}", flush=True)
    d = 128
    scale = float(np.float32(1.0 / np.sqrt(d)))
    cap = (max(lens) + ntok + 8 + bs - 1) // bs * bs
    bt = inputs.Batch(seed=7000 + k, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype="bf16", poison=True)
    rng = np.random.default_rng(8000 + k)
    lens_h = bt.lens.copy()
    max_len = int(lens_h.max())
    if form in ("attention", "step", "multi"):
        kc, vc = to_dev(bt.k_cache), to_dev(bt.v_cache)
        lens_d = torch.from_numpy(lens_h.copy()).cuda()
        kh, vh = bt.k_cache.copy(), bt.v_cache.copy()
        if form == "multi":
            q, kn, vn = (_draw(rng, (b, ntok, x, d)) for x in (h, g, g))
            ws = api.make_multi_workspace(b, ntok, h, g, d, d, torch.bfloat16, "cuda")
            out = torch.empty(b, ntok, h, d, dtype=torch.bfloat16, device="cuda")
            api.decode_step_multi(out, to_dev(q), to_dev(kn), to_dev(vn), kc, vc, lens_d, max_len, scale, ws)
            oracle_mod.kv_append_multi(kh, vh, kn, vn, lens_h)
            torch.cuda.synchronize()
            want = oracle_mod.decode_attention_multi(q, kh, vh, lens_h, scale)
        else:
            q = bt.q(0)
            ws = api.make_workspace(b, h, g, d, d, max_len + 1, torch.bfloat16, "cuda")
            out = torch.empty(b, h, d, dtype=torch.bfloat16, device="cuda")
            if form == "step":
                kn, vn = bt.new_kv(0)
                api.decode_step(out, to_dev(q), to_dev(kn), to_dev(vn), kc, vc, lens_d, max_len, scale, ws,
                                path=path, workgroups=wgs)
                oracle_mod.kv_append(kh, vh, kn, vn, lens_h)
            else:
                api.decode_attention(out, to_dev(q), kc, vc, lens_d, max_len, scale, ws, path=path, workgroups=wgs)
            torch.cuda.synchronize()
            want = oracle_mod.decode_attention(q, kh, vh, lens_h, scale)
            assert_counters_zero(ws, b, h)
        assert np.array_equal(lens_d.cpu().numpy(), lens_h)
        assert np.array_equal(to_host_bits(kc), kh) and np.array_equal(to_host_bits(vc), vh)
        assert_parity(out, want, "bf16", f"case {case}")
        return
    kp_h, table_h = make_paged(bt.k_cache, lens_h, bs, np.random.default_rng(9000 + k), room=ntok)
    vp_h, _ = make_paged(bt.v_cache, lens_h, bs, np.random.default_rng(9000 + k), room=ntok)
    kp, vp, table = to_dev(kp_h), to_dev(vp_h), torch.from_numpy(table_h).cuda()
    lens_d = torch.from_numpy(lens_h.copy()).cuda()
    if form == "multi_paged":
        q, kn, vn = (_draw(rng, (b, ntok, x, d)) for x in (h, g, g))
        ws = api.make_multi_workspace(b, ntok, h, g, d, d, torch.bfloat16, "cuda")
        out = torch.empty(b, ntok, h, d, dtype=torch.bfloat16, device="cuda")
        api.decode_step_multi_paged(out, to_dev(q), to_dev(kn), to_dev(vn), kp, vp, lens_d, table, max_len, scale, ws)
        torch.cuda.synchronize()
        oracle_mod.kv_append_multi_paged(kp_h, vp_h, kn, vn, lens_h, table_h)
        want = oracle_mod.decode_attention_multi_paged(q, kp_h, vp_h, lens_h, table_h, scale)
    else:
        q = bt.q(0)
        kn, vn = bt.new_kv(0)
        ws = api.make_workspace(b, h, g, d, d, max_len + 1, torch.bfloat16, "cuda")
        out = torch.empty(b, h, d, dtype=torch.bfloat16, device="cuda")
        api.decode_step_paged(out, to_dev(q), to_dev(kn), to_dev(vn), kp, vp, lens_d, table, max_len, scale, ws)
        torch.cuda.synchronize()
        oracle_mod.kv_append_paged(kp_h, vp_h, kn, vn, lens_h, table_h)
        want = oracle_mod.decode_attention_paged(q, kp_h, vp_h, lens_h, table_h, scale)
    assert np.array_equal(lens_d.cpu().numpy(), lens_h)
    assert np.array_equal(to_host_bits(kp), kp_h) and np.array_equal(to_host_bits(vp), vp_h)
    assert_parity(out, want, "bf16", f"case {case}")
