"""Pins of the oracle's projections and of its whole-layer decode step (CPU).

The projections follow the incremental-attention formulas of the MQA review
(§2.4: q, k, v are the token's vector contracted with P_q, P_k, P_v over the
model dimension, y is the attention output contracted with P_o over heads and
value dimensions; §3: P_k and P_v without the head axis). The oracle takes
the matrices output-major; these tests pin that layout against the pages'
einsum forms, against exact rational sums, and against closed forms, and pin
the layer's composition (projections held in the activation type, append
before attend, output projection of the attention result) against an
independent float64 restatement written with einsum.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from exact_round import round_bf16_exact
from gqa_kv_cache_decode_amd import inputs


def _bf16(a):
    return inputs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _f64(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def test_linear_matches_the_query_projection_einsum():
    # q[b,i,c] = sum_m x[b,m] P_q[i,m,c]; the oracle's W_q row i*d_k + c holds P_q[i,:,c]
    rng = np.random.default_rng(1)
    b, d_model, h, d_k = 3, 40, 4, 8
    x = _bf16(rng.standard_normal((b, d_model)))
    P = _bf16(rng.standard_normal((h, d_model, d_k)))
    W = np.ascontiguousarray(P.transpose(0, 2, 1).reshape(h * d_k, d_model))
    ref = np.einsum("bm,imc->bic", _f64(x), _f64(P))
    got = oracle.linear(x, W).reshape(b, h, d_k)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # rows ordered (c, i) instead of (i, c) would be a different map: the test can tell them apart
    W_other = np.ascontiguousarray(P.transpose(2, 0, 1).reshape(d_k * h, d_model))
    assert not np.allclose(oracle.linear(x, W_other).reshape(b, h, d_k), ref, rtol=1e-3, atol=1e-3)


def test_linear_matches_the_output_projection_einsum():
    # y[b,m] = sum_{i,c} o[b,i,c] P_o[i,m,c]; the oracle's W_o[m, i*d_v + c] = P_o[i,m,c]
    rng = np.random.default_rng(2)
    b, h, d_v, d_model = 2, 3, 8, 24
    o = _bf16(rng.standard_normal((b, h, d_v)))
    P = _bf16(rng.standard_normal((h, d_model, d_v)))
    W = np.ascontiguousarray(P.transpose(1, 0, 2).reshape(d_model, h * d_v))
    ref = np.einsum("bic,imc->bm", _f64(o), _f64(P))
    got = oracle.linear(np.ascontiguousarray(o.reshape(b, h * d_v)), W)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_linear_equals_exact_rational_sums():
    getcontext().prec = 60
    rng = np.random.default_rng(3)
    for rows, n_in, n_out in [(1, 1, 1), (2, 5, 3), (3, 16, 4)]:
        x = rng.standard_normal((rows, n_in)).astype(np.float32)
        w = rng.standard_normal((n_out, n_in)).astype(np.float32)
        got = oracle.linear(x, w)
        for r in range(rows):
            for o in range(n_out):
                exact = sum(Decimal(float(x[r, k])) * Decimal(float(w[o, k])) for k in range(n_in))
                assert abs(Decimal(got[r, o]) - exact) <= abs(exact) * Decimal(1e-14) + Decimal(1e-300)


def test_linear_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 6)).astype(np.float32)
    # identity weights give the input back exactly; a unit input picks a weight column
    assert np.array_equal(oracle.linear(x, np.eye(6, dtype=np.float32)), x.astype(np.float64))
    w = rng.standard_normal((5, 6)).astype(np.float32)
    e2 = np.zeros((1, 6), dtype=np.float32)
    e2[0, 2] = 1.0
    assert np.array_equal(oracle.linear(e2, w)[0], w[:, 2].astype(np.float64))
    # homogeneous: scaling x by a power of two scales y exactly
    assert np.array_equal(oracle.linear(np.float32(4.0) * x, w), 4.0 * oracle.linear(x, w))
    # each output row depends only on its own input row
    y = oracle.linear(x, w)
    assert np.array_equal(oracle.linear(np.ascontiguousarray(x[2:3]), w)[0], y[2])


def test_store_rounds_once_to_nearest():
    # the activation hold is one rounding of the fp64 value to the nearest
    # bf16 (ties to even), checked against exact rational rounding on values
    # with more significant bits than fp32 holds
    rng = np.random.default_rng(5)
    mant = 1.0 + rng.integers(0, 2 ** 40, 1500) * 2.0 ** -40
    vals = np.concatenate([
        rng.standard_normal(1500) * 10.0 ** rng.integers(-30, 30, 1500),
        mant * np.where(rng.random(1500) < 0.5, -1.0, 1.0) * 2.0 ** rng.integers(-120, 120, 1500),
        [0.0, -0.0, 1.0, -2.0, 1e-40, -3e-39],
    ])
    got = oracle.store(vals, np.uint16)
    want = np.array([round_bf16_exact(v) for v in vals], dtype=np.uint16)
    # a negative value that rounds to zero keeps its sign
    assert np.array_equal(got, want)
    # just above a tie that fp32 cannot hold: rounding through fp32 first would
    # land on the tie and go to even (0x3F80); one rounding goes up
    assert oracle.store(np.array([1 + 2.0 ** -8 + 2.0 ** -30]), np.uint16)[0] == 0x3F81
    assert oracle.store(np.array([1 + 2.0 ** -8]), np.uint16)[0] == 0x3F80      # exact tie: to even
    assert oracle.store(np.array([1 + 3 * 2.0 ** -8]), np.uint16)[0] == 0x3F82  # exact tie: to even
    assert oracle.store(np.array([np.inf, -np.inf, 3.4e38]), np.uint16).tolist() == [0x7F80, 0xFF80, 0x7F80]
    nan = oracle.store(np.array([np.nan]), np.uint16)[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    # fp32: numpy's conversion of a double is one correctly rounded step
    f32 = oracle.store(vals, np.float32)
    assert np.array_equal(f32, vals.astype(np.float32))


def _layer_by_einsum(x, P_q, P_k, P_v, P_o, k_cache, v_cache, lens, scale):
    """The layer step restated from the pages' einsum forms, in float64, each hold one exact rounding to bf16."""
    def hold(a):
        a = np.asarray(a, dtype=np.float64)
        return _f64(np.array([round_bf16_exact(v) for v in a.ravel()], dtype=np.uint16).reshape(a.shape))
    x = _f64(x)
    q = hold(np.einsum("bm,imc->bic", x, _f64(P_q)))
    k = hold(np.einsum("bm,jmc->bjc", x, _f64(P_k)))
    v = hold(np.einsum("bm,jmc->bjc", x, _f64(P_v)))
    K, V = _f64(k_cache), _f64(v_cache)
    b, g = K.shape[:2]
    h = q.shape[1]
    G = h // g
    attn = np.zeros((b, h, V.shape[3]))
    for s in range(b):
        L = int(lens[s])
        Ks = np.concatenate([K[s, :, :L], k[s, :, None]], axis=1)   # append, then attend
        Vs = np.concatenate([V[s, :, :L], v[s, :, None]], axis=1)
        for i in range(h):
            logit = scale * Ks[i // G] @ q[s, i]
            w = np.exp(logit - logit.max())
            attn[s, i] = (w / w.sum()) @ Vs[i // G]
    return np.einsum("bic,imc->bm", hold(attn), _f64(P_o))


@pytest.mark.parametrize("h,g", [(4, 2), (4, 4), (6, 1)])
def test_decode_layer_matches_an_einsum_restatement(h, g):
    rng = np.random.default_rng(6 + h + g)
    b, d_model, d, cap = 3, 32, 16, 12
    lens = np.array([0, 3, 10], dtype=np.int32)
    x = _bf16(rng.standard_normal((b, d_model)))
    P_q, P_k, P_v = (_bf16(rng.standard_normal(s) / np.sqrt(d_model)) for s in
                     [(h, d_model, d), (g, d_model, d), (g, d_model, d)])
    P_o = _bf16(rng.standard_normal((h, d_model, d)) / np.sqrt(h * d))
    k_cache = _bf16(rng.standard_normal((b, g, cap, d)))
    v_cache = _bf16(rng.standard_normal((b, g, cap, d)))
    scale = float(np.float32(1 / np.sqrt(d)))
    ref = _layer_by_einsum(x, P_q, P_k, P_v, P_o, k_cache, v_cache, lens, scale)

    W_q = np.ascontiguousarray(P_q.transpose(0, 2, 1).reshape(h * d, d_model))
    W_k = np.ascontiguousarray(P_k.transpose(0, 2, 1).reshape(g * d, d_model))
    W_v = np.ascontiguousarray(P_v.transpose(0, 2, 1).reshape(g * d, d_model))
    W_o = np.ascontiguousarray(P_o.transpose(1, 0, 2).reshape(d_model, h * d))
    kc, vc, ln = k_cache.copy(), v_cache.copy(), lens.copy()
    y, mid = oracle.decode_layer(x, W_q, W_k, W_v, W_o, kc, vc, ln, scale, h)
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)
    # the append: lengths grew by one, the new rows sit at the old lengths
    assert np.array_equal(ln, lens + 1)
    for s in range(b):
        assert np.array_equal(kc[s, :, lens[s]], mid["k_new"][s])
        assert np.array_equal(vc[s, :, lens[s]], mid["v_new"][s])
    # a sequence with nothing cached attends only to its own new token
    np.testing.assert_array_equal(mid["attn64"][0], np.repeat(_f64(mid["v_new"][0]), h // g, axis=0))
