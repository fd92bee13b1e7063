"""GPU append parity: the HIP append must equal the oracle's bit for bit.

Caches live inside larger buffers whose guard regions hold a fixed pattern;
the guards, every untouched slot (NaN-poisoned beyond the length) and the
lengths are compared exactly.
"""
import numpy as np
import pytest
import torch

from gpu_util import to_dev, to_host_bits, torch_dtype
from gqa_kv_cache_decode_amd import api, inputs
from gqa_kv_cache_decode_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements before and after each cache


def _guarded(arr: np.ndarray):
    """Device buffer [guard | arr | guard] and the contiguous view of arr inside it."""
    flat = np.ascontiguousarray(arr).reshape(-1)
    pat = (np.arange(GUARD) % 251).astype(arr.dtype) if arr.dtype == np.uint16 else \
        np.arange(GUARD, dtype=np.float32) * np.float32(-3.5)
    host = np.concatenate([pat, flat, pat])
    buf = to_dev(host)
    view = buf[GUARD:GUARD + flat.size].view(arr.shape)
    return buf, view, pat


def _check_guards(buf, pat, n):
    h = to_host_bits(buf)
    assert np.array_equal(h[:GUARD].view(np.uint8), pat.view(np.uint8)), "front guard overwritten"
    assert np.array_equal(h[GUARD + n:].view(np.uint8), pat.view(np.uint8)), "back guard overwritten"


def _run_append(name, steps=1, b_limit=None):
    wl = WORKLOADS[name]
    batch = inputs.Batch(seed=wl.seed, b=wl.b, h=wl.h, g=wl.g, d=wl.d, cap=wl.cap, lens=wl.lens,
                         dtype=wl.dtype, poison=True)
    return wl, batch


@pytest.mark.parametrize("name", ["tiny_gqa_f32", "mqa_bf16", "llama3_70b_gqa_bf16", "qwen25_7b_gqa_bf16"])
def test_append_bitwise(gpu_lib, oracle_mod, name):
    wl, batch = _run_append(name)
    print(f"append parity: {name}", flush=True)
    kbuf, kc, kpat = _guarded(batch.k_cache)
    vbuf, vc, vpat = _guarded(batch.v_cache)
    lens = torch.from_numpy(batch.lens.copy()).cuda()
    lens_h = batch.lens.copy()
    steps = min(wl.steps, 3)
    for step in range(steps):
        kn, vn = batch.new_kv(step)
        api.kv_append(kc, vc, to_dev(kn), to_dev(vn), lens, int(lens_h.max()))
        oracle_mod.kv_append(batch.k_cache, batch.v_cache, kn, vn, lens_h)
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), lens_h)
    assert np.array_equal(to_host_bits(kc).view(np.uint8), batch.k_cache.view(np.uint8))
    assert np.array_equal(to_host_bits(vc).view(np.uint8), batch.v_cache.view(np.uint8))
    _check_guards(kbuf, kpat, batch.k_cache.size)
    _check_guards(vbuf, vpat, batch.v_cache.size)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 256), ("bf16", 16), ("bf16", 64), ("f32", 12), ("bf16", 20)])
def test_append_shapes(gpu_lib, oracle_mod, dtype, d):
    b, g, cap = 5, 3, 40
    lens_h = np.array([0, 1, 17, 38, 39], np.int32)
    kc_h = inputs.draw_cache(31, inputs.TAG_K, b, g, cap, d, lens_h, dtype)
    vc_h = inputs.draw_cache(31, inputs.TAG_V, b, g, cap, d, lens_h, dtype)
    kbuf, kc, kpat = _guarded(kc_h)
    vbuf, vc, vpat = _guarded(vc_h)
    lens = torch.from_numpy(lens_h.copy()).cuda()
    kn, vn = inputs.draw_new_kv(31, 0, b, g, d, d, dtype)
    api.kv_append(kc, vc, to_dev(kn), to_dev(vn), lens, int(lens_h.max()))
    oracle_mod.kv_append(kc_h, vc_h, kn, vn, lens_h)
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), lens_h)
    assert np.array_equal(to_host_bits(kc).view(np.uint8), kc_h.view(np.uint8))
    assert np.array_equal(to_host_bits(vc).view(np.uint8), vc_h.view(np.uint8))
    _check_guards(kbuf, kpat, kc_h.size)
    _check_guards(vbuf, vpat, vc_h.size)


def test_append_full_sequence_left_untouched(gpu_lib):
    # A device length already at capacity violates the precondition; the
    # kernel writes nothing for that sequence and leaves its length alone.
    b, g, d, cap = 3, 2, 16, 8
    lens_h = np.array([2, 8, 5], np.int32)
    kc_h = inputs.draw_cache(32, inputs.TAG_K, b, g, cap, d, lens_h, "f32")
    vc_h = inputs.draw_cache(32, inputs.TAG_V, b, g, cap, d, lens_h, "f32")
    kc, vc = to_dev(kc_h), to_dev(vc_h)
    lens = torch.from_numpy(lens_h.copy()).cuda()
    kn, vn = inputs.draw_new_kv(32, 0, b, g, d, d, "f32")
    api.kv_append(kc, vc, to_dev(kn), to_dev(vn), lens, 5)  # host bound (wrong on purpose for s=1)
    torch.cuda.synchronize()
    got = lens.cpu().numpy()
    assert got.tolist() == [3, 8, 6]
    assert np.array_equal(to_host_bits(kc)[1].view(np.uint8), kc_h[1].view(np.uint8))
    assert np.array_equal(to_host_bits(kc)[0, :, 2], kn[0])
