"""Pin of the split-and-merge identity on the CPU (survey pin P9).

The oracle's chunked attention computes each chunk of positions on its own
(m_c, l_c, o_c) and combines them with the softmax over a union of position
sets (MQA review §2.1): out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
In exact arithmetic this is the direct softmax; in fp64 the two forms must
agree to within a few units of rounding (1e-13 relative here) for every way
of cutting the positions, including empty chunks, one position per chunk and
logits far from zero. This is the identity the GPU's split-K schedule relies
on when a segment is shared by several workgroups.
"""
import numpy as np
import pytest

import oracle
from gqa_kv_cache_decode_amd import inputs


def _random_bounds(rng, lens, n_chunks):
    b = len(lens)
    bounds = np.zeros((b, n_chunks + 1), dtype=np.int32)
    for s, L in enumerate(lens):
        cuts = np.sort(rng.integers(0, L + 1, n_chunks - 1)) if n_chunks > 1 else np.array([], dtype=np.int64)
        bounds[s, 1:-1] = cuts
        bounds[s, -1] = L
    return bounds


def _close(a, b, rel=1e-13):
    scale = max(float(np.abs(b).max(initial=0.0)), 1e-300)
    return float(np.abs(a - b).max(initial=0.0)) <= rel * scale


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("h,g", [(4, 2), (6, 3), (8, 1), (5, 5)])
def test_chunked_equals_direct_for_random_cuts(dtype, h, g):
    rng = np.random.default_rng(900 + h * 10 + g)
    lens = [0, 1, 7, 40, 129]
    batch = inputs.Batch(seed=901 + h + g, b=len(lens), h=h, g=g, d=8, cap=130, lens=lens, dtype=dtype, poison=False)
    q = batch.q(0)
    scale = float(np.float32(1 / np.sqrt(8)))
    direct = oracle.decode_attention(q, batch.k_cache, batch.v_cache, batch.lens, scale)
    for n_chunks in (1, 2, 3, 5, 8, 17):
        bounds = _random_bounds(rng, lens, n_chunks)
        got = oracle.decode_attention_chunked(q, batch.k_cache, batch.v_cache, batch.lens, bounds, scale)
        assert _close(got, direct), (n_chunks, np.abs(got - direct).max())


def test_one_position_per_chunk_and_large_logits():
    # the finest cut, with logits of several hundred (exp(s) alone would overflow)
    lens = [3, 50]
    batch = inputs.Batch(seed=911, b=2, h=4, g=2, d=16, cap=50, lens=lens, dtype="f32", poison=False)
    q = batch.q(0) * np.float32(30.0)
    direct = oracle.decode_attention(q, batch.k_cache, batch.v_cache, batch.lens, 1.0)
    n = max(lens)
    bounds = np.array([[min(t, L) for t in range(n + 1)] for L in lens], dtype=np.int32)
    got = oracle.decode_attention_chunked(q, batch.k_cache, batch.v_cache, batch.lens, bounds, 1.0)
    assert np.isfinite(got).all()
    assert _close(got, direct)


def test_the_rescale_matters():
    # cutting where the maximum moves: combining the chunks without the
    # e^(m_c - M) factors would be far off, the merge is not
    lens = [64]
    batch = inputs.Batch(seed=912, b=1, h=2, g=1, d=16, cap=64, lens=lens, dtype="f32", poison=False)
    q = batch.q(0) * np.float32(8.0)
    bounds = np.array([[0, 10, 33, 64]], dtype=np.int32)
    direct = oracle.decode_attention(q, batch.k_cache, batch.v_cache, batch.lens, 1.0)
    got = oracle.decode_attention_chunked(q, batch.k_cache, batch.v_cache, batch.lens, bounds, 1.0)
    assert _close(got, direct)
    # each chunk's own normalised output differs from the whole
    part = oracle.decode_attention(q, batch.k_cache, batch.v_cache, np.array([10], dtype=np.int32), 1.0)
    assert np.abs(part - direct).max() > 1e-3


def test_bad_bounds_are_rejected():
    batch = inputs.Batch(seed=913, b=1, h=2, g=1, d=8, cap=8, lens=[5], dtype="f32", poison=False)
    q = batch.q(0)
    for bad in ([[1, 5]], [[0, 4]], [[0, 3, 2, 5]]):
        with pytest.raises(oracle.OracleError):
            oracle.decode_attention_chunked(q, batch.k_cache, batch.v_cache, batch.lens, np.array(bad), 1.0)
