"""Pins of the oracle's multi-token calls over paged caches (CPU).

The paged multi-token append and attention stand for the contiguous
multi-token ones on the cache the pool stands for (row t of KV head j of
sequence s is pool[table[s][t // B]][j][t % B]). Pinned here: the append of
n tokens that crosses block boundaries equals the contiguous multi-token
append read back through the gather, bit for bit, and touches no other pool
row; the attention equals the contiguous multi-token attention bit for bit
and does not change when blocks move around the pool; a sequence without
room for its n tokens, or a needed table entry that names no block, changes
nothing.
"""
import numpy as np
import pytest

import oracle
from gqa_kv_cache_decode_amd import inputs
from paged_util import make_paged


def _setup(seed, n, lens=(0, 30, 61), b=3, h=8, g=2, d=16, cap=128, bs=32, dtype="bf16"):
    bt = inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=list(lens), dtype=dtype, poison=True)
    rng = np.random.default_rng(seed)
    kp, table = make_paged(bt.k_cache, bt.lens, bs, rng, room=n)
    vp, _ = make_paged(bt.v_cache, bt.lens, bs, np.random.default_rng(seed), room=n)

    def draw(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x
    return bt, kp, vp, table, draw((b, n, h, d)), draw((b, n, g, d)), draw((b, n, g, d))


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("n,dtype", [(4, "bf16"), (3, "f32"), (1, "bf16")])
def test_append_crossing_blocks_equals_the_contiguous_append(n, dtype):
    bt, kp, vp, table, q, kn, vn = _setup(61 + n, n, dtype=dtype)   # 30 + 3/4 and 61 + 3/4 cross a 32-row block
    lens_p = bt.lens.copy()
    kp0 = kp.copy()
    oracle.kv_append_multi_paged(kp, vp, kn, vn, lens_p, table)
    kc, vc, lens_c = bt.k_cache.copy(), bt.v_cache.copy(), bt.lens.copy()
    oracle.kv_append_multi(kc, vc, kn, vn, lens_c)
    assert np.array_equal(lens_p, lens_c) and np.array_equal(lens_p, bt.lens + n)
    cap = bt.k_cache.shape[2]
    for pool, want in ((kp, kc), (vp, vc)):
        got = oracle.gather_paged(pool, table, lens_p, 32, cap)
        for s in range(3):
            assert np.array_equal(_bits(got[s, :, :lens_p[s]]), _bits(want[s, :, :lens_p[s]]))
    # rows outside the appended slots are untouched (NaN poison included)
    changed = np.zeros(kp.shape[:3], dtype=bool)
    for s in range(3):
        for t in range(bt.lens[s], bt.lens[s] + n):
            changed[table[s, t // 32], :, t % 32] = True
    assert np.array_equal(_bits(kp[~changed]), _bits(kp0[~changed]))


@pytest.mark.parametrize("h,g,n", [(8, 2, 4), (8, 8, 2), (6, 1, 3)])
def test_attention_equals_the_contiguous_attention_and_ignores_block_placement(h, g, n):
    bt, kp, vp, table, q, kn, vn = _setup(71 + h + g + n, n, h=h, g=g)
    lens = bt.lens.copy()
    oracle.kv_append_multi_paged(kp, vp, kn, vn, lens, table)
    got = oracle.decode_attention_multi_paged(q, kp, vp, lens, table, 0.25)
    kc, vc, lens_c = bt.k_cache.copy(), bt.v_cache.copy(), bt.lens.copy()
    oracle.kv_append_multi(kc, vc, kn, vn, lens_c)
    want = oracle.decode_attention_multi(q, kc, vc, lens_c, 0.25)
    assert np.array_equal(got, want)
    # move every block to another place in the pool: same result
    perm = np.random.default_rng(5).permutation(kp.shape[0])
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    assert np.array_equal(oracle.decode_attention_multi_paged(q, kp2, vp2, lens, table2, 0.25), want)


def test_no_room_or_bad_entry_changes_nothing():
    bt, kp, vp, table, q, kn, vn = _setup(81, 4, lens=(0, 30, 125))   # 125 + 4 > 128
    lens = bt.lens.copy()
    kp0, vp0 = kp.copy(), vp.copy()
    with pytest.raises(oracle.OracleError) as e:
        oracle.kv_append_multi_paged(kp, vp, kn, vn, lens, table)
    assert e.value.code == oracle.ERR_CAPACITY
    assert np.array_equal(lens, bt.lens) and np.array_equal(kp, kp0) and np.array_equal(vp, vp0)
    bt, kp, vp, table, q, kn, vn = _setup(82, 4, lens=(0, 30, 61))
    table[1, 1] = -1                                                   # positions 32.. of sequence 1
    lens = bt.lens.copy()
    kp0 = kp.copy()
    with pytest.raises(oracle.OracleError) as e:
        oracle.kv_append_multi_paged(kp, vp, kn, vn, lens, table)
    assert e.value.code == oracle.ERR_ARG
    assert np.array_equal(lens, bt.lens) and np.array_equal(kp, kp0)
