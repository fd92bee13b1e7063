"""Pins of the oracle's paged-cache functions (CPU).

A paged cache stands for the contiguous cache whose row t of KV head j of
sequence s is pool[table[s][t // B]][j][t % B] (the reading taken for the
block-table caches the pages name without a layout). These tests pin the
gather against numpy fancy indexing and against the one-block-per-sequence
case (which is the contiguous cache itself), the paged append against the
contiguous append, and the attention over a pool against the attention over
the cache it stands for, including invariance under moving blocks around
the pool and never reading poisoned spare blocks or rows.
"""
import numpy as np
import pytest

import oracle
from gqa_kv_cache_decode_amd import inputs
from paged_util import make_paged


def _batch(seed, b=3, h=8, g=2, d=16, cap=100, lens=(0, 37, 99), dtype="bf16"):
    return inputs.Batch(seed=seed, b=b, h=h, g=g, d=d, cap=cap, lens=list(lens), dtype=dtype, poison=True)


@pytest.mark.parametrize("block_size", [32, 64, 128])
def test_gather_matches_fancy_indexing(block_size):
    rng = np.random.default_rng(block_size)
    bt = _batch(501)
    pool, table = make_paged(bt.k_cache, bt.lens, block_size, rng)
    got = oracle.gather_paged(pool, table, bt.lens, block_size, bt.k_cache.shape[2])
    for s in range(3):
        t = np.arange(bt.lens[s])
        want = pool[table[s, t // block_size], :, t % block_size].transpose(1, 0, 2)  # [g, L, d]
        assert np.array_equal(got[s, :, :bt.lens[s]], want)
        assert np.array_equal(got[s, :, :bt.lens[s]], bt.k_cache[s, :, :bt.lens[s]])
        assert np.all(got[s, :, bt.lens[s]:] == 0)


def test_one_block_per_sequence_is_the_contiguous_cache():
    bt = _batch(502, cap=96, lens=(0, 37, 95))
    pool = np.ascontiguousarray(bt.k_cache)               # block s = sequence s, B = cap
    table = np.arange(3, dtype=np.int32).reshape(3, 1)
    got = oracle.gather_paged(pool, table, bt.lens, 96, 96)
    for s in range(3):
        assert np.array_equal(got[s, :, :bt.lens[s]], bt.k_cache[s, :, :bt.lens[s]])


def test_paged_append_equals_contiguous_append():
    rng = np.random.default_rng(3)
    bt = _batch(503, lens=(0, 63, 64))
    kp, table = make_paged(bt.k_cache, bt.lens, 32, rng)
    vp, _ = make_paged(bt.v_cache, bt.lens, 32, np.random.default_rng(3))
    kn, vn = bt.new_kv(0)
    lens_p = bt.lens.copy()
    oracle.kv_append_paged(kp, vp, kn, vn, lens_p, table)
    kc, vc, lens_c = bt.k_cache.copy(), bt.v_cache.copy(), bt.lens.copy()
    oracle.kv_append(kc, vc, kn, vn, lens_c)
    assert np.array_equal(lens_p, lens_c)
    cap = bt.k_cache.shape[2]
    for got, want in ((oracle.gather_paged(kp, table, lens_p, 32, cap), kc),
                      (oracle.gather_paged(vp, table, lens_p, 32, cap), vc)):
        for s in range(3):
            assert np.array_equal(got[s, :, :lens_p[s]], want[s, :, :lens_p[s]])
    # positions 63 -> 64 cross into a new block: the new row is row 0 of block table[s][2]
    assert np.array_equal(kp[table[2, 2], :, 0], kn[2])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_over_a_pool_is_the_attention_over_its_cache(dtype):
    rng = np.random.default_rng(4)
    bt = _batch(504, h=8, g=2, dtype=dtype, lens=(1, 70, 100))
    scale = 0.25
    kp, table = make_paged(bt.k_cache, bt.lens, 32, rng)
    vp, _ = make_paged(bt.v_cache, bt.lens, 32, np.random.default_rng(4))
    q = bt.q(0)
    want = oracle.decode_attention(q, bt.k_cache, bt.v_cache, bt.lens, scale)
    got = oracle.decode_attention_paged(q, kp, vp, bt.lens, table, scale)
    assert np.array_equal(got, want)
    assert np.isfinite(got).all()  # spare blocks and rows past the lengths are NaN and never read
    # move every block elsewhere in the pool (and fix the table): the output does not change
    perm = rng.permutation(kp.shape[0])
    inv = np.argsort(perm)
    table2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1).astype(np.int32)
    got2 = oracle.decode_attention_paged(q, np.ascontiguousarray(kp[perm]), np.ascontiguousarray(vp[perm]),
                                         bt.lens, table2, scale)
    assert np.array_equal(got2, want)


def test_paged_errors():
    bt = _batch(505, lens=(0, 31, 64))
    kp, table = make_paged(bt.k_cache, bt.lens, 32, np.random.default_rng(5), room=0)
    vp, _ = make_paged(bt.v_cache, bt.lens, 32, np.random.default_rng(5), room=0)
    kn, vn = bt.new_kv(0)
    # without room for the append, sequence 0 (empty) has no block and sequence 2 (64 rows)
    # would need a third one: the table holds -1 there
    lens = bt.lens.copy()
    with pytest.raises(oracle.OracleError) as e:
        oracle.kv_append_paged(kp, vp, kn, vn, lens, table)
    assert e.value.code == oracle.ERR_ARG
    assert np.array_equal(lens, bt.lens)  # nothing changed
    kp, table = make_paged(bt.k_cache, bt.lens, 32, np.random.default_rng(5), room=1)
    vp, _ = make_paged(bt.v_cache, bt.lens, 32, np.random.default_rng(5), room=1)
    full = bt.lens.copy()
    full[1] = table.shape[1] * 32
    with pytest.raises(oracle.OracleError) as e:
        oracle.kv_append_paged(kp, vp, kn, vn, full, table)
    assert e.value.code == oracle.ERR_CAPACITY
    bad = table.copy()
    bad[1, 0] = kp.shape[0]
    with pytest.raises(oracle.OracleError) as e:
        oracle.gather_paged(kp, bad, bt.lens, 32, 100)
    assert e.value.code == oracle.ERR_ARG
