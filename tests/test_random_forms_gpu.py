"""Parity over randomly drawn shapes (seeded; the same cases every run) for
the call forms beyond the one-token contiguous step: paged one-token
attention and fused step, multi-token attention over contiguous caches, and
multi-token append + attention over paged caches. Element type, head dim,
KV heads, heads per group, new tokens, block size and ragged lengths vary
together; outputs are held to the decode parity bar against the fp64
oracle, appended rows and lengths bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, to_dev, to_host_bits
from gqa_kv_cache_decode_amd import api, inputs
from paged_util import make_paged

pytestmark = pytest.mark.gpu

FORMS = ("paged_attention", "paged_step", "multi", "multi_paged")


def _cases(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        form = FORMS[k % len(FORMS)]
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        d = int(rng.choice([16, 64, 128, 128, 128, 256]))
        g = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 32]))
        n = int(rng.choice([2, 3, 4, 8])) if form.startswith("multi") else 1
        while n * g * G > 512:
            G = max(1, G // 2)
        b = int(rng.integers(1, 10))
        lens = rng.integers(0, 400, b)
        if not form.startswith("multi"):
            lens[rng.random(b) < 0.15] = 0
        bs = int(rng.choice([32, 64, 256]))
        out.append((k, form, dtype, b, g * G, g, d, n, [int(x) for x in lens], bs))
    return out


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-{c[1]}")
def test_random_form(gpu_lib, oracle_mod, case):
    k, form, dtype, b, h, g, d, n, lens, bs = case
    print(f"random form {case}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = float(np.float32(1.0 / np.sqrt(d)))
    cap = (max(lens) + n + 8 + bs - 1) // bs * bs
    bt = inputs.Batch(seed=4000 + k, b=b, h=h, g=g, d=d, cap=cap, lens=lens, dtype=dtype, poison=True)
    rng = np.random.default_rng(5000 + k)
    lens_h = bt.lens.copy()
    max_len = int(lens_h.max())
    if form == "multi":
        q, kn, vn = (_draw(rng, (b, n, x, d), dtype) for x in (h, g, g))
        kc, vc = to_dev(bt.k_cache), to_dev(bt.v_cache)
        lens_d = torch.from_numpy(lens_h.copy()).cuda()
        ws = api.make_multi_workspace(b, n, h, g, d, d, tdt, "cuda")
        out = torch.empty(b, n, h, d, dtype=tdt, device="cuda")
        api.decode_step_multi(out, to_dev(q), to_dev(kn), to_dev(vn), kc, vc, lens_d, max_len, scale, ws)
        torch.cuda.synchronize()
        kh, vh = bt.k_cache.copy(), bt.v_cache.copy()
        oracle_mod.kv_append_multi(kh, vh, kn, vn, lens_h)
        assert np.array_equal(lens_d.cpu().numpy(), lens_h)
        assert np.array_equal(_bits(to_host_bits(kc)), _bits(kh)) and np.array_equal(_bits(to_host_bits(vc)), _bits(vh))
        want = oracle_mod.decode_attention_multi(q, kh, vh, lens_h, scale)
        assert_parity(out, want, dtype, f"case {case}")
        return
    kp_h, table_h = make_paged(bt.k_cache, lens_h, bs, np.random.default_rng(6000 + k), room=n)
    vp_h, _ = make_paged(bt.v_cache, lens_h, bs, np.random.default_rng(6000 + k), room=n)
    kp, vp, table = to_dev(kp_h), to_dev(vp_h), torch.from_numpy(table_h).cuda()
    lens_d = torch.from_numpy(lens_h.copy()).cuda()
    if form == "multi_paged":
        q, kn, vn = (_draw(rng, (b, n, x, d), dtype) for x in (h, g, g))
        ws = api.make_multi_workspace(b, n, h, g, d, d, tdt, "cuda")
        out = torch.empty(b, n, h, d, dtype=tdt, device="cuda")
        api.decode_step_multi_paged(out, to_dev(q), to_dev(kn), to_dev(vn), kp, vp, lens_d, table, max_len, scale, ws)
        torch.cuda.synchronize()
        oracle_mod.kv_append_multi_paged(kp_h, vp_h, kn, vn, lens_h, table_h)
        want = oracle_mod.decode_attention_multi_paged(q, kp_h, vp_h, lens_h, table_h, scale)
    else:
        q = bt.q(0)
        ws = api.make_workspace(b, h, g, d, d, max_len + 1, tdt, "cuda")
        out = torch.empty(b, h, d, dtype=tdt, device="cuda")
        if form == "paged_step":
            kn, vn = bt.new_kv(0)
            api.decode_step_paged(out, to_dev(q), to_dev(kn), to_dev(vn), kp, vp, lens_d, table, max_len, scale, ws)
            oracle_mod.kv_append_paged(kp_h, vp_h, kn, vn, lens_h, table_h)
        else:
            api.decode_attention_paged(out, to_dev(q), kp, vp, lens_d, table, max(max_len, 0), scale, ws)
        torch.cuda.synchronize()
        want = oracle_mod.decode_attention_paged(q, kp_h, vp_h, lens_h, table_h, scale)
    assert np.array_equal(lens_d.cpu().numpy(), lens_h)
    assert np.array_equal(_bits(to_host_bits(kp)), _bits(kp_h)) and np.array_equal(_bits(to_host_bits(vp)), _bits(vp_h))
    assert_parity(out, want, dtype, f"case {case}")
