"""Pins of the oracle's KV-head mean-fold and of its once-rounding to bf16 (CPU).

The TF2 GQA lesson turns a trained multi-head model into a grouped one by
averaging the key/value heads of each contiguous group, and its lab then runs
the three variants at the same weights: with g = h nothing may differ from
MHA, with fewer KV heads the output must change. The fold here is that mean,
taken over the heads of a cache (or of a key/value projection, which is the
same contraction before the projection is applied). These tests pin it
against exact rational arithmetic (the mean and its rounding), against
closed forms (one head per group, equal heads, nested folds), against the
lesson's g = h rule, and against the grouped attention it feeds.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_round import bf16_bits, bf16_value, frac_round
from gqa_kv_cache_decode_amd import inputs


_frac_round, _bf16_bits, _bf16_value = frac_round, bf16_bits, bf16_value


def test_round_bf16_is_a_single_rounding():
    rng = np.random.default_rng(21)
    vals = np.concatenate([rng.standard_normal(400) * 10.0 ** rng.integers(-40, 39, 400),
                           rng.standard_normal(100) * 1e-39])
    got = oracle.round_bf16(vals)
    for v, g in zip(vals, got):
        want = _frac_round(Fraction(float(v)), 8, -126, 127)
        zero_sign = 0x8000 if (want == 0 and v < 0) else 0  # a negative value that rounds to zero is -0
        assert g == (_bf16_bits(want) | zero_sign), v
    # a value just above a bf16 tie that fp32 cannot hold: rounding through fp32 first
    # would land on the tie and go to even (1.0); once-rounding goes up
    assert oracle.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81
    assert oracle.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 0x3F80          # exact tie: to even
    assert oracle.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82      # exact tie: to even
    assert oracle.round_bf16(np.array([-0.0]))[0] == 0x8000
    assert oracle.round_bf16(np.array([2.0 ** -133]))[0] == 0x0001           # smallest subnormal
    assert oracle.round_bf16(np.array([2.0 ** -134]))[0] == 0x0000           # tie to even zero
    assert oracle.round_bf16(np.array([3.4e38]))[0] == 0x7F80                 # past the largest: inf
    nan = oracle.round_bf16(np.array([np.nan]))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


@pytest.mark.parametrize("g_src,g_dst", [(4, 2), (6, 2), (5, 1), (12, 4), (8, 8), (7, 7), (6, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_equals_the_exact_mean_rounded_once(g_src, g_dst, dtype):
    rng = np.random.default_rng(100 + g_src * 10 + g_dst)
    b, cap, d = 2, 3, 4
    vals = rng.standard_normal((b, g_src, cap, d)) * 10.0 ** rng.integers(-6, 6, (b, g_src, cap, d))
    src = inputs.f32_to_bf16_bits(vals.astype(np.float32)) if dtype == "bf16" else vals.astype(np.float32)
    got = oracle.fold_heads(src, g_dst)
    F = g_src // g_dst
    for s in range(b):
        for j in range(g_dst):
            for t in range(cap):
                for c in range(d):
                    heads = range(j * F, (j + 1) * F)
                    if dtype == "bf16":
                        mean = sum(_bf16_value(src[s, i, t, c]) for i in heads) / F
                        assert got[s, j, t, c] == _bf16_bits(_frac_round(mean, 8, -126, 127))
                    else:
                        mean = sum(Fraction(float(src[s, i, t, c])) for i in heads) / F
                        assert Fraction(float(got[s, j, t, c])) == _frac_round(mean, 24, -126, 127)


def test_fold_sums_in_double_and_rounds_once():
    # heads 4, 2^-6, 2^-28, 0: the mean is 1 + 2^-8 + 2^-30, just above a bf16 tie. A sum
    # in fp32, or rounding the mean through fp32, lands on the tie and goes to even (1.0).
    vals = np.array([4.0, 2.0 ** -6, 2.0 ** -28, 0.0], dtype=np.float32)
    src = np.ascontiguousarray(np.broadcast_to(inputs.f32_to_bf16_bits(vals)[None, :, None, None], (1, 4, 1, 8)))
    assert np.all(oracle.fold_heads(src, 1) == 0x3F81)


def test_one_head_per_group_is_a_copy_and_rows_past_the_length_stay():
    rng = np.random.default_rng(22)
    src = inputs.f32_to_bf16_bits(rng.standard_normal((3, 4, 9, 8)).astype(np.float32))
    lens = np.array([0, 4, 9], dtype=np.int32)
    out = np.full((3, 4, 12, 8), 0xABCD, dtype=np.uint16)
    oracle.fold_heads(src, 4, lens, out=out)
    for s in range(3):
        assert np.array_equal(out[s, :, :lens[s]], src[s, :, :lens[s]])
        assert np.all(out[s, :, lens[s]:] == 0xABCD)


def test_equal_heads_fold_to_themselves_and_opposite_heads_to_zero():
    rng = np.random.default_rng(23)
    one = rng.standard_normal((2, 1, 5, 8)).astype(np.float32)
    same = np.ascontiguousarray(np.repeat(one, 6, axis=1))
    assert np.array_equal(oracle.fold_heads(same, 2), np.repeat(one, 2, axis=1))
    pm = np.ascontiguousarray(np.concatenate([one, -one], axis=1))
    assert np.array_equal(oracle.fold_heads(pm, 1), np.zeros_like(one))


def test_nested_folds_compose_in_exact_arithmetic():
    # small integers: every sum and every quotient by a power of two is exact
    rng = np.random.default_rng(24)
    src = rng.integers(-64, 64, (2, 16, 5, 8)).astype(np.float32)
    direct = oracle.fold_heads(src, 2)
    nested = oracle.fold_heads(oracle.fold_heads(src, 8), 2)
    assert np.array_equal(direct, nested)
    assert np.array_equal(direct, src.reshape(2, 2, 8, 5, 8).mean(axis=2))


def test_fold_picks_contiguous_groups():
    # head i holds the constant i: contiguous groups of F average to jF + (F - 1)/2
    b, g_src, cap, d = 1, 12, 2, 8
    src = np.broadcast_to(np.arange(g_src, dtype=np.float32)[None, :, None, None], (b, g_src, cap, d)).copy()
    for g_dst in (1, 2, 3, 4, 6):
        F = g_src // g_dst
        got = oracle.fold_heads(src, g_dst)
        assert np.array_equal(got[0, :, 0, 0], np.array([j * F + (F - 1) / 2 for j in range(g_dst)], np.float32))


def test_fold_of_the_key_projection_is_the_fold_of_the_keys():
    # k = x W_k^T; W_k [g*d][d_model] folded as b = 1, cap = d, width d_model gives the
    # projection whose keys are the folded keys (exact with small-integer operands)
    rng = np.random.default_rng(25)
    g, d, d_model, rows = 8, 4, 16, 3
    W = rng.integers(-8, 8, (g * d, d_model)).astype(np.float32)
    x = rng.integers(-8, 8, (rows, d_model)).astype(np.float32)
    Wf = oracle.fold_heads(W.reshape(1, g, d, d_model), 2).reshape(2 * d, d_model)
    k = oracle.linear(x, W).astype(np.float32).reshape(1, rows, g, d).transpose(0, 2, 1, 3)
    k_folded = oracle.fold_heads(np.ascontiguousarray(k), 2)
    assert np.array_equal(oracle.linear(x, Wf).reshape(rows, 2, d), k_folded[0].transpose(1, 0, 2))


def test_fold_feeds_the_grouped_attention():
    rng = np.random.default_rng(26)
    b, h, cap, d = 2, 8, 6, 16
    lens = np.array([3, 6], dtype=np.int32)
    K = inputs.f32_to_bf16_bits(rng.standard_normal((b, h, cap, d)).astype(np.float32))
    V = inputs.f32_to_bf16_bits(rng.standard_normal((b, h, cap, d)).astype(np.float32))
    q = inputs.f32_to_bf16_bits(rng.standard_normal((b, h, d)).astype(np.float32))
    scale = 0.25
    mha = oracle.decode_attention(q, K, V, lens, scale)
    # g = h: the fold is the identity and the output is MHA's, bit for bit
    assert np.array_equal(oracle.decode_attention(q, oracle.fold_heads(K, h, lens), oracle.fold_heads(V, h, lens),
                                                  lens, scale), mha)
    for g in (4, 2, 1):
        Kf, Vf = oracle.fold_heads(K, g, lens), oracle.fold_heads(V, g, lens)
        gqa = oracle.decode_attention(q, Kf, Vf, lens, scale)
        # the grouped call equals MHA over the folded heads repeated per query head
        rep = oracle.decode_attention(q, np.ascontiguousarray(np.repeat(Kf, h // g, axis=1)),
                                      np.ascontiguousarray(np.repeat(Vf, h // g, axis=1)), lens, scale)
        assert np.array_equal(gqa, rep)
        # and, at the same weights, fewer KV heads change the output
        assert np.abs(gqa - mha).max() > 1e-3


def test_fold_errors():
    src = np.zeros((1, 6, 4, 8), dtype=np.float32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.fold_heads(src, 4)
    assert e.value.code == oracle.ERR_GROUPS
    with pytest.raises(oracle.OracleError) as e:
        oracle.fold_heads(src, 3, max_rows=5)
    assert e.value.code == oracle.ERR_CAPACITY
    with pytest.raises(oracle.OracleError) as e:
        oracle.fold_heads(src, 3, np.array([5], dtype=np.int32))
    assert e.value.code == oracle.ERR_CAPACITY
