"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic. Both sides of every parity check (the HIP library and
the CPU oracle) consume the arrays it returns.

Recipe:

* Every block of values has its own PCG64 stream keyed by
  ``SeedSequence(seed, spawn_key=(tag, *index))``, so any block (one KV head
  of one sequence, the query of one step, ...) can be redrawn on its own and
  blocks can be drawn in parallel threads.
* Values are ``standard_normal`` float32. For bf16 workloads they are rounded
  to bf16 with round-to-nearest-even and returned as raw uint16 bit patterns.
* Cache slots at or beyond a sequence's length are filled with NaN
  (``poison=True``, the default for correctness runs) or zero, so that a
  kernel that reads past the length shows up as NaN.
* Lengths are either a fixed value or integers drawn uniformly from an
  inclusive range.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

# spawn-key tags, one per kind of block
TAG_LENS = 1
TAG_K = 2
TAG_V = 3
TAG_Q = 4
TAG_KNEW = 5
TAG_VNEW = 6
TAG_X = 7        # the token vectors entering a layer
TAG_WEIGHT = 8   # projection matrices (key: which matrix, then the row block)

BF16_NAN = np.uint16(0x7FC0)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normals(seed: int, key: tuple, n: int, dtype: str) -> np.ndarray:
    """n standard normals from the stream (seed, key), as float32 or bf16 bits."""
    v = _rng(seed, *key).standard_normal(n, dtype=np.float32)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16}[dtype]


def draw_lens(seed: int, b: int, spec) -> np.ndarray:
    """Pre-append cache lengths: an int, a list of ints, or ("uniform", lo, hi) inclusive."""
    if isinstance(spec, int):
        return np.full(b, spec, dtype=np.int32)
    if isinstance(spec, (list, tuple)) and spec and spec[0] == "uniform":
        _, lo, hi = spec
        return _rng(seed, TAG_LENS).integers(lo, hi + 1, size=b, dtype=np.int64).astype(np.int32)
    arr = np.asarray(spec, dtype=np.int32)
    if arr.shape != (b,):
        raise ValueError("explicit lens must have one entry per sequence")
    return arr.copy()


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_cache(seed: int, tag: int, b: int, g: int, cap: int, d: int, lens: np.ndarray,
               dtype: str, poison: bool = True) -> np.ndarray:
    """One cache tensor [b, g, cap, d]: normals in slots < lens[b], NaN (or 0) beyond."""
    sd = storage_dtype(dtype)
    out = np.empty((b, g, cap, d), dtype=sd)

    def fill(bj):
        s, j = bj
        n = int(lens[s])
        if n > cap:
            raise ValueError("length exceeds capacity")
        if n:
            out[s, j, :n, :] = normals(seed, (tag, s, j), n * d, dtype).reshape(n, d)
        if n < cap:
            if poison:
                out[s, j, n:, :] = (np.float32(np.nan) if dtype == "f32" else BF16_NAN)
            else:
                out[s, j, n:, :] = 0

    jobs = [(s, j) for s in range(b) for j in range(g)]
    if len(jobs) * cap * d < (1 << 20):
        for job in jobs:
            fill(job)
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, jobs))
    return out


def draw_q(seed: int, step: int, b: int, h: int, d: int, dtype: str) -> np.ndarray:
    """Query of one decode step, [b, h, d]."""
    return normals(seed, (TAG_Q, step), b * h * d, dtype).reshape(b, h, d)


def draw_new_kv(seed: int, step: int, b: int, g: int, d_k: int, d_v: int, dtype: str):
    """The K and V rows appended at one decode step, [b, g, d_k] and [b, g, d_v]."""
    k = normals(seed, (TAG_KNEW, step), b * g * d_k, dtype).reshape(b, g, d_k)
    v = normals(seed, (TAG_VNEW, step), b * g * d_v, dtype).reshape(b, g, d_v)
    return k, v


def draw_x(seed: int, step: int, b: int, d_model: int, dtype: str) -> np.ndarray:
    """The token vectors entering a layer at one decode step, [b, d_model]."""
    return normals(seed, (TAG_X, step), b * d_model, dtype).reshape(b, d_model)


def draw_weight(seed: int, which: int, n_out: int, n_in: int, dtype: str) -> np.ndarray:
    """A projection matrix [n_out, n_in] with entries N(0, 1/n_in) (rows drawn in parallel blocks).

    which: 0 query, 1 key, 2 value, 3 output projection.
    """
    std = np.float32(1.0 / np.sqrt(n_in))
    rows_per = max(1, (1 << 20) // n_in)
    blocks = [(r0, min(n_out, r0 + rows_per)) for r0 in range(0, n_out, rows_per)]
    out = np.empty((n_out, n_in), dtype=storage_dtype(dtype))

    def fill(blk):
        r0, r1 = blk
        v = _rng(seed, TAG_WEIGHT, which, r0).standard_normal((r1 - r0) * n_in, dtype=np.float32) * std
        out[r0:r1] = (v if dtype == "f32" else f32_to_bf16_bits(v)).reshape(r1 - r0, n_in)

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, blocks))
    return out


class Batch:
    """All host arrays of one decode problem, before the append of step 0."""

    def __init__(self, *, seed, b, h, g, d, cap, lens, dtype, poison=True):
        self.seed, self.b, self.h, self.g, self.d, self.cap = seed, b, h, g, d, cap
        self.dtype = dtype
        self.lens = draw_lens(seed, b, lens)
        if int(self.lens.max(initial=0)) > cap:
            raise ValueError("a drawn length exceeds the capacity")
        self.k_cache = draw_cache(seed, TAG_K, b, g, cap, d, self.lens, dtype, poison)
        self.v_cache = draw_cache(seed, TAG_V, b, g, cap, d, self.lens, dtype, poison)

    def q(self, step: int) -> np.ndarray:
        return draw_q(self.seed, step, self.b, self.h, self.d, self.dtype)

    def new_kv(self, step: int):
        return draw_new_kv(self.seed, step, self.b, self.g, self.d, self.d, self.dtype)
