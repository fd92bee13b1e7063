"""fp64 CPU oracle for the GQA/MQA KV-cache decode step.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers. The product path
(``gqa_kv_cache_decode_amd``) never imports this package, and this package
never imports the product's code; the two share only the seeded input
generator, which holds none of the method's arithmetic.

The arithmetic lives in ``gqa_oracle.c`` (plain loops in double precision,
compiled with ``gcc -O2 -fopenmp -ffp-contract=off``). This module is
marshalling only: numpy arrays in, numpy arrays out.

Pages the oracle follows (cited by title and section):

* [MQA-review] velog review of "Fast Transformer Decoding: One Write-Head is
  All You Need": §2.1 Dot-Product Attention (the k contraction, softmax and
  v contraction), §2.4 Multi-head Attention (Incremental) (new K/V row
  concatenated on the position axis, then attention over all rows), §3 Multi
  Query Attention (K/V lose the head axis).
* [GQA-lesson] ttlab "TF2 GQA" lesson: the g-knob table, the h mod g = 0 rule,
  the cache element-count formula, the multiplication counts and the lab
  description (contiguous query-head groups; K/V repeated per query head).
* [LLM-inf-05] albangk "LLM inference 05" notes: the prefill/decode table, the
  per-layer decode pseudocode and the bytes-per-token arithmetic.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_golden.py``, ``tests/test_oracle_layer.py``,
``tests/test_oracle_fold.py``, ``tests/test_oracle_paged.py``,
``tests/test_oracle_multi.py``, ``tests/test_oracle_multi_paged.py`` and
``tests/test_oracle_merge.py`` (no function is "parity unpinned").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_gqa.so")

F32 = 0
BF16 = 1

OK = 0
ERR_ARG = -1
ERR_GROUPS = -2
ERR_UNSUPPORTED = -3
ERR_CAPACITY = -4


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def build() -> str:
    """Compile the C oracle in place (always recompiles)."""
    cmd = [
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
        "-std=c99", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    i32 = ctypes.c_int
    i64 = ctypes.c_int64
    lib.oracle_kv_cache_elems.restype = i64
    lib.oracle_kv_cache_elems.argtypes = [i64, i64, i64, i64]
    lib.oracle_kv_bytes_per_token.restype = i64
    lib.oracle_kv_bytes_per_token.argtypes = [i64, i64, i64, i64]
    lib.oracle_kv_append.restype = i32
    lib.oracle_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32]
    lib.oracle_decode_attention.restype = i32
    lib.oracle_decode_attention.argtypes = [
        vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
        ctypes.c_float, i32, vp, i32,
    ]
    lib.oracle_decode_attention_chunked.restype = i32
    lib.oracle_decode_attention_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                    ctypes.c_float, i32, i32]
    lib.oracle_linear.restype = i32
    lib.oracle_linear.argtypes = [vp, vp, vp, i32, i32, i32, i32]
    lib.oracle_store.restype = None
    lib.oracle_store.argtypes = [vp, vp, ctypes.c_size_t, i32]
    lib.oracle_fold_heads.restype = i32
    lib.oracle_fold_heads.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.oracle_round_bf16.restype = None
    lib.oracle_round_bf16.argtypes = [vp, vp, ctypes.c_size_t]
    lib.oracle_gather_paged.restype = i32
    lib.oracle_gather_paged.argtypes = [vp, vp, vp, vp] + [i32] * 8
    lib.oracle_kv_append_paged.restype = i32
    lib.oracle_kv_append_paged.argtypes = [vp] * 6 + [i32] * 8
    lib.oracle_kv_append_multi.restype = i32
    lib.oracle_kv_append_multi.argtypes = [vp] * 5 + [i32] * 7
    _lib = lib
    return lib


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {arr.dtype}")


def _ptr(arr: np.ndarray):
    return arr.ctypes.data_as(ctypes.c_void_p)


def kv_cache_elems(layers: int, kv_heads: int, length: int, head_dim: int) -> int:
    """2 x layers x KV heads x length x head dim [GQA-lesson]."""
    return int(_load().oracle_kv_cache_elems(layers, kv_heads, length, head_dim))


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes one token adds to a model's cache [LLM-inf-05, memory arithmetic]."""
    return int(_load().oracle_kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes))


def kv_append(k_cache, v_cache, k_new, v_new, lens) -> None:
    """In place: write each sequence's new K/V row at position lens[b], then lens[b] += 1.

    k_cache [b, g, cap, d_k], v_cache [b, g, cap, d_v], k_new [b, g, d_k],
    v_new [b, g, d_v], lens int32 [b]; all C-contiguous numpy arrays of one
    element type (float32, or uint16 bf16 bit patterns).
    """
    for a in (k_cache, v_cache, k_new, v_new, lens):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    if lens.dtype != np.int32:
        raise TypeError("lens must be int32")
    b, g, cap, d_k = k_cache.shape
    d_v = v_cache.shape[3]
    dt = _dtype_code(k_cache)
    rc = _load().oracle_kv_append(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(lens),
        b, g, d_k, d_v, cap, dt)
    if rc != OK:
        raise OracleError(rc, "kv_append")


def decode_attention(q, k_cache, v_cache, lens, scale: float, *, want_weights=False,
                     threads: int = 0, count_muls=False):
    """Attention of one query token per sequence against its cache, in fp64.

    q [b, h, d_k]; caches [b, g, cap, d]; lens int32 [b] (attended lengths).
    Returns out [b, h, d_v] float64, plus weights [b, h, cap] float64 and/or
    the multiplication count when asked.
    """
    for a in (q, k_cache, v_cache, lens):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    if lens.dtype != np.int32:
        raise TypeError("lens must be int32")
    b, h, d_k = q.shape
    bk, g, cap, dk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if bk != b or dk2 != d_k or v_cache.shape[:3] != (b, g, cap):
        raise ValueError("shape mismatch between q and caches")
    dt = _dtype_code(k_cache)
    if _dtype_code(q) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("q, K and V must share an element type")
    out = np.empty((b, h, d_v), dtype=np.float64)
    weights = np.empty((b, h, cap), dtype=np.float64) if want_weights else None
    muls = ctypes.c_int64(0)
    rc = _load().oracle_decode_attention(
        _ptr(out), _ptr(weights) if weights is not None else None,
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
        b, h, g, d_k, d_v, cap, ctypes.c_float(scale), dt,
        ctypes.byref(muls) if count_muls else None, threads)
    if rc != OK:
        raise OracleError(rc, "decode_attention")
    res = [out]
    if want_weights:
        res.append(weights)
    if count_muls:
        res.append(int(muls.value))
    return res[0] if len(res) == 1 else tuple(res)


def decode_attention_chunked(q, k_cache, v_cache, lens, bounds, scale: float, threads: int = 0) -> np.ndarray:
    """decode_attention computed chunk by chunk and merged [MQA-review §2.1 softmax over a union of chunks].

    bounds int32 [b, n_chunks + 1]: chunk c of sequence s is positions
    bounds[s, c] .. bounds[s, c + 1] - 1 (0 first, lens[s] last, non-decreasing).
    """
    for a in (q, k_cache, v_cache, lens):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    bounds = np.ascontiguousarray(bounds, dtype=np.int32)
    b, h, d_k = q.shape
    _, g, cap, _ = k_cache.shape
    d_v = v_cache.shape[3]
    if bounds.ndim != 2 or bounds.shape[0] != b:
        raise OracleError(ERR_ARG, "decode_attention_chunked bounds")
    dt = _dtype_code(k_cache)
    out = np.empty((b, h, d_v), dtype=np.float64)
    rc = _load().oracle_decode_attention_chunked(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(np.ascontiguousarray(lens, dtype=np.int32)),
        _ptr(bounds), bounds.shape[1] - 1, b, h, g, d_k, d_v, cap, ctypes.c_float(scale), dt, threads)
    if rc != OK:
        raise OracleError(rc, "decode_attention_chunked")
    return out


def linear(x, w) -> np.ndarray:
    """y[r][o] = sum_k x[r][k] * w[o][k] in fp64 [MQA-review §2.4 projections].

    x [rows, n_in], w [n_out, n_in] (output-major), same element type.
    """
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    dt = _dtype_code(x)
    if _dtype_code(w) != dt or x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise OracleError(ERR_ARG, "linear shapes")
    y = np.zeros((x.shape[0], w.shape[0]), dtype=np.float64)
    rc = _load().oracle_linear(_ptr(y), _ptr(x), _ptr(w), x.shape[0], x.shape[1], w.shape[0], dt)
    if rc != OK:
        raise OracleError(rc, "linear")
    return y


def store(values, like_dtype) -> np.ndarray:
    """Hold fp64 values in an element type (float32, or bf16 bit patterns as uint16), nearest even."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    dt = F32 if np.dtype(like_dtype) == np.float32 else BF16
    out = np.empty(values.shape, dtype=np.float32 if dt == F32 else np.uint16)
    _load().oracle_store(_ptr(out), _ptr(values), values.size, dt)
    return out


def decode_layer(x, w_q, w_k, w_v, w_o, k_cache, v_cache, lens, scale: float, h: int):
    """One decode step of a layer [MQA-review §2.4 incremental attention; §3 for g = 1].

    q = x W_q^T, k_new = x W_k^T, v_new = x W_v^T (each held in the activation
    type), append (k_cache, v_cache and lens updated in place), attention of q
    over the grown caches (held in the activation type), then y = attn W_o^T.
    Returns (y fp64 [b, d_model], dict of the intermediate arrays).
    """
    b = x.shape[0]
    g, d_k, d_v = k_cache.shape[1], k_cache.shape[3], v_cache.shape[3]
    q = store(linear(x, w_q), x.dtype).reshape(b, h, d_k)
    k_new = store(linear(x, w_k), x.dtype).reshape(b, g, d_k)
    v_new = store(linear(x, w_v), x.dtype).reshape(b, g, d_v)
    kv_append(k_cache, v_cache, k_new, v_new, lens)
    attn64 = decode_attention(q, k_cache, v_cache, lens, scale)
    attn = store(attn64, x.dtype)
    y = linear(attn.reshape(b, h * d_v), w_o)
    return y, {"q": q, "k_new": k_new, "v_new": v_new, "attn": attn, "attn64": attn64}


def round_bf16(values) -> np.ndarray:
    """fp64 values rounded once to bf16 (nearest even), as uint16 bit patterns."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=np.uint16)
    _load().oracle_round_bf16(_ptr(out), _ptr(values), values.size)
    return out


def fold_heads(src, g_dst: int, lens=None, *, out=None, max_rows=None) -> np.ndarray:
    """Mean-fold of contiguous groups of KV heads [GQA-lesson, merging the groups].

    src [b, g_src, cap, d] (float32 or bf16 bits); lens int32 [b] (rows per
    sequence) or None (all max_rows rows, default cap). Returns dst [b, g_dst,
    cap_dst, d]: ``out`` if given (rows at or beyond each length untouched),
    else a new zero array of src's capacity.
    """
    src = np.ascontiguousarray(src)
    b, g_src, cap_src, d = src.shape
    dt = _dtype_code(src)
    if out is None:
        out = np.zeros((b, g_dst, cap_src, d), dtype=src.dtype)
    if not out.flags.c_contiguous or out.dtype != src.dtype or out.shape[0] != b or out.shape[1] != g_dst \
            or out.shape[3] != d:
        raise OracleError(ERR_ARG, "fold_heads output")
    if lens is not None:
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        if lens.shape != (b,):
            raise OracleError(ERR_ARG, "fold_heads lens")
    rows = int(max_rows) if max_rows is not None else (int(lens.max()) if lens is not None else cap_src)
    rc = _load().oracle_fold_heads(_ptr(out), _ptr(src), _ptr(lens) if lens is not None else None, b, g_src,
                                   g_dst, cap_src, out.shape[2], d, rows, dt)
    if rc != OK:
        raise OracleError(rc, "fold_heads")
    return out


def gather_paged(pool, table, lens, block_size: int, cap: int) -> np.ndarray:
    """The contiguous cache [b, g, cap, d] a paged pool stands for (rows t < lens[s]; zeros after).

    pool [num_blocks, g, block_size, d]; table int32 [b, max_blocks]: row t of
    head j of sequence s is pool[table[s, t // block_size], j, t % block_size].
    """
    pool = np.ascontiguousarray(pool)
    table = np.ascontiguousarray(table, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    num_blocks, g, bs, d = pool.shape
    if bs != block_size or table.ndim != 2 or lens.shape != (table.shape[0],):
        raise OracleError(ERR_ARG, "gather_paged shapes")
    b, max_blocks = table.shape
    out = np.zeros((b, g, cap, d), dtype=pool.dtype)
    rc = _load().oracle_gather_paged(_ptr(out), _ptr(pool), _ptr(table), _ptr(lens), b, g, block_size, max_blocks,
                                     num_blocks, cap, d, _dtype_code(pool))
    if rc != OK:
        raise OracleError(rc, "gather_paged")
    return out


def kv_append_paged(k_pool, v_pool, k_new, v_new, lens, table) -> None:
    """In place: each sequence's new rows go to position lens[s] of its paged cache; lens += 1."""
    for a in (k_pool, v_pool, k_new, v_new, lens, table):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    if lens.dtype != np.int32 or table.dtype != np.int32:
        raise TypeError("lens and table must be int32")
    num_blocks, g, bs, d_k = k_pool.shape
    d_v = v_pool.shape[3]
    b, max_blocks = table.shape
    rc = _load().oracle_kv_append_paged(_ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new), _ptr(lens),
                                        _ptr(table), b, g, d_k, d_v, bs, max_blocks, num_blocks,
                                        _dtype_code(k_pool))
    if rc != OK:
        raise OracleError(rc, "kv_append_paged")


def decode_attention_paged(q, k_pool, v_pool, lens, table, scale: float, **kw):
    """Attention over paged caches: the attention of decode_attention over the caches they stand for."""
    bs = k_pool.shape[2]
    cap = table.shape[1] * bs
    k = gather_paged(k_pool, table, lens, bs, cap)
    v = gather_paged(v_pool, table, lens, bs, cap)
    return decode_attention(q, k, v, np.ascontiguousarray(lens, dtype=np.int32), scale, **kw)


def kv_append_multi(k_cache, v_cache, k_new, v_new, lens) -> None:
    """In place: token r of sequence s goes to position lens[s] + r; lens += n.

    k_new [b, n, g, d_k], v_new [b, n, g, d_v] [MQA-review §2.3 batched positions, §2.4].
    """
    for a in (k_cache, v_cache, k_new, v_new, lens):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    if lens.dtype != np.int32:
        raise TypeError("lens must be int32")
    b, g, cap, d_k = k_cache.shape
    d_v = v_cache.shape[3]
    n = k_new.shape[1]
    if k_new.shape != (b, n, g, d_k) or v_new.shape != (b, n, g, d_v):
        raise OracleError(ERR_ARG, "kv_append_multi shapes")
    rc = _load().oracle_kv_append_multi(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(lens),
                                        b, n, g, d_k, d_v, cap, _dtype_code(k_cache))
    if rc != OK:
        raise OracleError(rc, "kv_append_multi")


def decode_attention_multi(q, k_cache, v_cache, lens, scale: float, threads: int = 0) -> np.ndarray:
    """n query tokens per sequence over a cache that already holds them, with the causal mask.

    q [b, n, h, d_k]; lens int32 [b] = attended length of the last token (the n new
    tokens are the positions lens[s] - n .. lens[s] - 1). Token r attends positions
    t < lens[s] - (n - 1 - r): everything before it and itself [MQA-review §2.3, the
    batched form whose additive mask removes later positions; LLM-inf-05: under the
    causal mask a position's K and V depend only on the positions up to it]. Each
    token's row is the single-token attention over its own prefix. Returns [b, n, h, d_v].
    """
    b, n, h, d_k = q.shape
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if np.any(lens < n):
        raise OracleError(ERR_ARG, "decode_attention_multi: every length must include the n new tokens")
    out = np.empty((b, n, h, v_cache.shape[3]), dtype=np.float64)
    for r in range(n):
        prefix = (lens - (n - 1 - r)).astype(np.int32)
        out[:, r] = decode_attention(np.ascontiguousarray(q[:, r]), k_cache, v_cache, prefix, scale, threads=threads)
    return out


def kv_append_multi_paged(k_pool, v_pool, k_new, v_new, lens, table) -> None:
    """In place: token r of sequence s goes to position lens[s] + r of its paged cache; lens += n.

    The multi-token append (n single appends in a row [MQA-review §2.3, §2.4])
    on the block-table layout of kv_append_paged. All or nothing: if any
    sequence lacks room for its n tokens or a table entry they need is not a
    pool block, nothing changes (OracleError).
    """
    b, n, g, d_k = k_new.shape
    num_blocks, _, bs, _ = k_pool.shape
    max_blocks = table.shape[1]
    for s in range(b):
        L = int(lens[s])
        if L < 0 or L + n > max_blocks * bs:
            raise OracleError(ERR_CAPACITY, "kv_append_multi_paged")
        for t in range(L, L + n):
            if not 0 <= int(table[s, t // bs]) < num_blocks:
                raise OracleError(ERR_ARG, "kv_append_multi_paged: table entry")
    for r in range(n):
        kv_append_paged(k_pool, v_pool, np.ascontiguousarray(k_new[:, r]), np.ascontiguousarray(v_new[:, r]), lens,
                        table)


def decode_attention_multi_paged(q, k_pool, v_pool, lens, table, scale: float, threads: int = 0) -> np.ndarray:
    """Multi-token causal attention over paged caches: decode_attention_multi over the caches they stand for."""
    bs = k_pool.shape[2]
    cap = table.shape[1] * bs
    k = gather_paged(k_pool, table, lens, bs, cap)
    v = gather_paged(v_pool, table, lens, bs, cap)
    return decode_attention_multi(q, k, v, np.ascontiguousarray(lens, dtype=np.int32), scale, threads=threads)
