"""Thin torch binding over the C ABI of include/gqa_decode.h.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and sizes go to libgqa_decode.so on
torch's current stream (or the stream given). Every step of the decode path
runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import MERGE_INLINE, MERGE_KERNEL, MERGE_SPREAD, PATH_AUTO, PATH_MATRIX, PATH_VECTOR  # noqa: F401  (re-exported)

_DTYPES = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype}; use float32 or bfloat16") from None


# torch's raw handle of the current stream, without building a Stream object
# (a few microseconds per call, which matter for steps of ~20 us)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_gpu(*tensors: torch.Tensor) -> None:
    dev = tensors[0].get_device()  # -1 for host tensors
    for t in tensors:
        if t.get_device() != dev or not t.is_cuda:
            raise ValueError("all tensors must live on the same GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    # the library launches on the current device (and its current stream)
    if dev != torch.cuda.current_device():
        raise ValueError(f"tensors live on cuda:{dev}, the current device is cuda:{torch.cuda.current_device()} "
                         "(use torch.cuda.device or torch.cuda.set_device)")


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, lens: torch.Tensor, max_len: int, stream=None) -> None:
    """Store k_new [b,g,d_k] / v_new [b,g,d_v] at slot lens[s] of each sequence; lens += 1.

    max_len: host-side upper bound of lens before the call.
    """
    _check_gpu(k_cache, v_cache, k_new, v_new, lens)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    b, g, cap, d_k = k_cache.shape
    d_v = v_cache.shape[3]
    if tuple(v_cache.shape) != (b, g, cap, d_v) or tuple(k_new.shape) != (b, g, d_k) \
            or tuple(v_new.shape) != (b, g, d_v) or tuple(lens.shape) != (b,):
        raise ValueError("kv_append: inconsistent shapes")
    dt = _dtype_code(k_cache)
    if any(_dtype_code(t) != dt for t in (v_cache, k_new, v_new)):
        raise TypeError("caches and new rows must share one element type")
    lib = _lib.load()
    rc = lib.gqa_kv_append(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(),
                           v_new.data_ptr(), lens.data_ptr(), b, g, d_k, d_v, cap, int(max_len),
                           dt, _stream_handle(stream))
    _lib.check(rc, "gqa_kv_append")


def workspace_size(b: int, h: int, g: int, d_k: int, d_v: int, max_len: int, dtype: torch.dtype) -> int:
    n = _lib.load().gqa_decode_workspace_size(b, h, g, d_k, d_v, int(max_len), _DTYPES[dtype])
    if n == 0:
        raise ValueError("gqa_decode_workspace_size rejected the shape")
    return int(n)


def make_workspace(b: int, h: int, g: int, d_k: int, d_v: int, max_len: int, dtype: torch.dtype,
                   device) -> torch.Tensor:
    """A zero-filled workspace (the library keeps its counters zero between calls)."""
    return torch.zeros(workspace_size(b, h, g, d_k, d_v, max_len, dtype), dtype=torch.uint8, device=device)


def plan(b, h, g, d_k, d_v, cap, max_len, dtype: torch.dtype, path=PATH_AUTO, workgroups=0, stream_flag=False):
    """(path, workgroups, merge) the library would launch with on the current device; no GPU work.

    path is PATH_VECTOR or PATH_MATRIX; merge is MERGE_INLINE, MERGE_KERNEL or MERGE_SPREAD. With
    stream_flag, a fourth value says whether the matrix path runs its one-block
    streaming kernel.
    """
    lib = _lib.load()
    p, c = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib.gqa_decode_plan(b, h, g, d_k, d_v, cap, int(max_len), _DTYPES[dtype], path, workgroups,
                             ctypes.byref(p), ctypes.byref(c))
    _lib.check(rc, "gqa_decode_plan")
    merge = p.value & (MERGE_INLINE | MERGE_KERNEL | MERGE_SPREAD)
    chosen = p.value & ~(MERGE_INLINE | MERGE_KERNEL | MERGE_SPREAD | _lib.PLAN_STREAM)
    if stream_flag:
        return chosen, c.value, merge, bool(p.value & _lib.PLAN_STREAM)
    return chosen, c.value, merge


def decode_attention(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     lens: torch.Tensor, max_len: int, scale: float, workspace: torch.Tensor,
                     path: int = PATH_AUTO, workgroups: int = 0, stream=None) -> torch.Tensor:
    """out[s,i] = softmax_t(scale * q[s,i] . K[s,j,t]) @ V[s,j,t], t < lens[s], j = i // (h/g).

    q [b,h,d_k], caches [b,g,cap,d], lens int32 [b] (attended lengths), out [b,h,d_v].
    path: PATH_* optionally OR-ed with MERGE_INLINE / MERGE_KERNEL / MERGE_SPREAD.
    """
    _check_gpu(out, q, k_cache, v_cache, lens, workspace)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    b, h, d_k = q.shape
    bk, g, cap, dk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if bk != b or dk2 != d_k or tuple(v_cache.shape) != (b, g, cap, d_v) \
            or tuple(out.shape) != (b, h, d_v) or tuple(lens.shape) != (b,):
        raise ValueError("decode_attention: inconsistent shapes")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_cache, v_cache, out)):
        raise TypeError("q, caches and out must share one element type")
    lib = _lib.load()
    rc = lib.gqa_decode_attention_ex(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(),
        b, h, g, d_k, d_v, cap, int(max_len), ctypes.c_float(scale), dt,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream),
        path, workgroups)
    _lib.check(rc, "gqa_decode_attention")
    return out


def decode_step(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor, lens: torch.Tensor, max_len: int, scale: float,
                workspace: torch.Tensor, path: int = PATH_AUTO, workgroups: int = 0, stream=None) -> torch.Tensor:
    """Append k_new/v_new at slot lens[s], attend over [0, lens[s] + 1), then lens += 1 — one launch.

    max_len: host-side upper bound of lens before the call.
    """
    _check_gpu(out, q, k_new, v_new, k_cache, v_cache, lens, workspace)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    b, h, d_k = q.shape
    bk, g, cap, dk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if bk != b or dk2 != d_k or tuple(v_cache.shape) != (b, g, cap, d_v) or tuple(out.shape) != (b, h, d_v) \
            or tuple(lens.shape) != (b,) or tuple(k_new.shape) != (b, g, d_k) or tuple(v_new.shape) != (b, g, d_v):
        raise ValueError("decode_step: inconsistent shapes")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_cache, v_cache, out, k_new, v_new)):
        raise TypeError("q, rows, caches and out must share one element type")
    lib = _lib.load()
    rc = lib.gqa_decode_step_ex(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        lens.data_ptr(), b, h, g, d_k, d_v, cap, int(max_len), ctypes.c_float(scale), dt,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream), path, workgroups)
    _lib.check(rc, "gqa_decode_step")
    return out


def decode_step_static(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       k_cache: torch.Tensor, v_cache: torch.Tensor, lens: torch.Tensor, max_len: int, scale: float,
                       stream=None) -> torch.Tensor:
    """decode_step with the library's own per-GPU scratch array as workspace (allocates nothing).

    Calls that overlap on one GPU race on that array; serialise them.
    """
    _check_gpu(out, q, k_new, v_new, k_cache, v_cache, lens)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    b, h, d_k = q.shape
    bk, g, cap, dk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if bk != b or dk2 != d_k or tuple(v_cache.shape) != (b, g, cap, d_v) or tuple(out.shape) != (b, h, d_v) \
            or tuple(lens.shape) != (b,) or tuple(k_new.shape) != (b, g, d_k) or tuple(v_new.shape) != (b, g, d_v):
        raise ValueError("decode_step_static: inconsistent shapes")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_cache, v_cache, out, k_new, v_new)):
        raise TypeError("q, rows, caches and out must share one element type")
    lib = _lib.load()
    rc = lib.gqa_decode_step_static(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        lens.data_ptr(), b, h, g, d_k, d_v, cap, int(max_len), ctypes.c_float(scale), dt, _stream_handle(stream))
    _lib.check(rc, "gqa_decode_step_static")
    return out


class PackedWeight:
    """A [n_out, n_in] bf16 weight matrix in the library's packed layout (gqa_pack_weight)."""

    def __init__(self, w: torch.Tensor, stream=None):
        _check_gpu(w)
        if w.dim() != 2 or w.dtype != torch.bfloat16:
            raise ValueError("PackedWeight takes a 2-d bfloat16 matrix [n_out, n_in]")
        self.n_out, self.n_in = w.shape
        lib = _lib.load()
        nbytes = int(lib.gqa_packed_weight_bytes(self.n_out, self.n_in))
        self.data = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
        _lib.check(lib.gqa_pack_weight(self.data.data_ptr(), w.data_ptr(), self.n_out, self.n_in, _lib.BF16,
                                       _stream_handle(stream)), "gqa_pack_weight")


def linear(y: torch.Tensor, x: torch.Tensor, w: PackedWeight, stream=None) -> torch.Tensor:
    """y[r] = W @ x[r] for a decode batch: x [rows, n_in], W [n_out, n_in] packed, y [rows, n_out], bf16."""
    _check_gpu(y, x, w.data)
    rows, n_in = x.shape
    if w.n_in != n_in or tuple(y.shape) != (rows, w.n_out):
        raise ValueError("linear: inconsistent shapes")
    dt = _dtype_code(x)
    if _dtype_code(y) != dt:
        raise TypeError("x and y must share one element type")
    rc = _lib.load().gqa_linear(y.data_ptr(), x.data_ptr(), w.data.data_ptr(), rows, n_in, w.n_out, dt,
                                _stream_handle(stream))
    _lib.check(rc, "gqa_linear")
    return y


class LayerScratch:
    """Device buffers for the intermediate results of decode_layer (q, k_new, v_new, attn)."""

    def __init__(self, b: int, h: int, g: int, d_k: int, d_v: int, dtype: torch.dtype, device):
        self.q = torch.empty(b, h, d_k, dtype=dtype, device=device)
        self.k_new = torch.empty(b, g, d_k, dtype=dtype, device=device)
        self.v_new = torch.empty(b, g, d_v, dtype=dtype, device=device)
        self.attn = torch.empty(b, h, d_v, dtype=dtype, device=device)


def decode_layer(y: torch.Tensor, x: torch.Tensor, w_q: PackedWeight, w_k: PackedWeight, w_v: PackedWeight,
                 w_o: PackedWeight, k_cache: torch.Tensor, v_cache: torch.Tensor, lens: torch.Tensor, max_len: int,
                 scale: float, workspace: torch.Tensor, scratch: LayerScratch, stream=None) -> torch.Tensor:
    """Projections, append, attention and output projection of one decode step (gqa_decode_layer).

    x, y [b, d_model]; packed w_q [h*d_k, d_model], w_k [g*d_k, d_model], w_v [g*d_v, d_model],
    w_o [d_model, h*d_v]; caches [b, g, cap, d]; lens int32 [b] (pre-append, grows by one).
    """
    _check_gpu(y, x, w_q.data, w_k.data, w_v.data, w_o.data, k_cache, v_cache, lens, workspace, scratch.q,
               scratch.k_new, scratch.v_new, scratch.attn)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    b, d_model = x.shape
    bk, g, cap, d_k = k_cache.shape
    d_v = v_cache.shape[3]
    h = scratch.q.shape[1]
    shape = lambda w: (w.n_out, w.n_in)  # noqa: E731
    if bk != b or tuple(y.shape) != (b, d_model) or shape(w_q) != (h * d_k, d_model) \
            or shape(w_k) != (g * d_k, d_model) or shape(w_v) != (g * d_v, d_model) \
            or shape(w_o) != (d_model, h * d_v) or tuple(v_cache.shape) != (b, g, cap, d_v) \
            or tuple(scratch.q.shape) != (b, h, d_k) or tuple(scratch.k_new.shape) != (b, g, d_k) \
            or tuple(scratch.v_new.shape) != (b, g, d_v) or tuple(scratch.attn.shape) != (b, h, d_v) \
            or tuple(lens.shape) != (b,):
        raise ValueError("decode_layer: inconsistent shapes")
    dt = _dtype_code(x)
    if any(_dtype_code(t) != dt for t in (y, k_cache, v_cache, scratch.q)):
        raise TypeError("activations and caches must share one element type")
    rc = _lib.load().gqa_decode_layer(
        y.data_ptr(), x.data_ptr(), w_q.data.data_ptr(), w_k.data.data_ptr(), w_v.data.data_ptr(),
        w_o.data.data_ptr(),
        scratch.q.data_ptr(), scratch.k_new.data_ptr(), scratch.v_new.data_ptr(), scratch.attn.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(), b, h, g, d_model, d_k, d_v, cap, int(max_len),
        ctypes.c_float(scale), dt, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_handle(stream))
    _lib.check(rc, "gqa_decode_layer")
    return y


def fold_kv_heads(dst: torch.Tensor, src: torch.Tensor, lens: torch.Tensor | None = None,
                  max_rows: int | None = None, stream=None) -> torch.Tensor:
    """Mean-fold of contiguous KV-head groups (C entry point gqa_fold_kv_heads).

    src [b, g_src, cap_src, d] -> dst [b, g_dst, cap_dst, d], same dtype; rows t < lens[s]
    (or < max_rows, default the smaller capacity, when lens is None).
    """
    _check_gpu(dst, src)
    if src.dim() != 4 or dst.dim() != 4 or src.shape[0] != dst.shape[0] or src.shape[3] != dst.shape[3]:
        raise ValueError("fold_kv_heads: src [b, g_src, cap, d] and dst [b, g_dst, cap, d] expected")
    b, g_src, cap_src, d = src.shape
    g_dst, cap_dst = dst.shape[1], dst.shape[2]
    dt = _dtype_code(src)
    if _dtype_code(dst) != dt:
        raise TypeError("src and dst must share one element type")
    lens_ptr = None
    if lens is not None:
        _check_gpu(lens)
        if lens.dtype != torch.int32 or tuple(lens.shape) != (b,):
            raise ValueError("lens must be int32 [b]")
        lens_ptr = lens.data_ptr()
    rows = min(cap_src, cap_dst) if max_rows is None else int(max_rows)
    rc = _lib.load().gqa_fold_kv_heads(dst.data_ptr(), src.data_ptr(), lens_ptr, b, g_src, g_dst, cap_src, cap_dst,
                                       d, rows, dt, _stream_handle(stream))
    _lib.check(rc, "gqa_fold_kv_heads")
    return dst


def read_bandwidth(src: torch.Tensor, sink: torch.Tensor, stream=None) -> torch.Tensor:
    """Read every byte of src once (C entry point gqa_read_bandwidth), one workgroup per sink word.

    src: any contiguous device tensor whose byte size is a multiple of 16; sink: int32 [workgroups],
    receiving each workgroup's sum of the 32-bit words it read (mod 2^32).
    """
    _check_gpu(src, sink)
    if sink.dtype != torch.int32 or sink.dim() != 1:
        raise ValueError("sink must be int32 [workgroups]")
    rc = _lib.load().gqa_read_bandwidth(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                        sink.numel(), _stream_handle(stream))
    _lib.check(rc, "gqa_read_bandwidth")
    return sink


def _paged_args(k_pool: torch.Tensor, v_pool: torch.Tensor, table: torch.Tensor, lens: torch.Tensor):
    _check_gpu(k_pool, v_pool, table, lens)
    if table.dtype != torch.int32 or lens.dtype != torch.int32 or table.dim() != 2:
        raise TypeError("block table [b, max_blocks] and lens [b] must be int32")
    num_blocks, g, bs, d_k = k_pool.shape
    if tuple(v_pool.shape[:3]) != (num_blocks, g, bs):
        raise ValueError("k_pool and v_pool must share [num_blocks, g, block_size]")
    b, max_blocks = table.shape
    if tuple(lens.shape) != (b,):
        raise ValueError("lens must be [b]")
    return b, g, d_k, v_pool.shape[3], bs, max_blocks, num_blocks


def kv_append_paged(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    lens: torch.Tensor, block_table: torch.Tensor, max_len: int, stream=None) -> None:
    """Store k_new / v_new [b, g, d] at position lens[s] of each paged cache; lens += 1."""
    b, g, d_k, d_v, bs, mb, nb = _paged_args(k_pool, v_pool, block_table, lens)
    _check_gpu(k_pool, k_new, v_new)
    if tuple(k_new.shape) != (b, g, d_k) or tuple(v_new.shape) != (b, g, d_v):
        raise ValueError("kv_append_paged: k_new [b, g, d_k] and v_new [b, g, d_v] expected")
    if any(_dtype_code(t) != _dtype_code(k_pool) for t in (v_pool, k_new, v_new)):
        raise TypeError("pools and new rows must share one element type")
    rc = _lib.load().gqa_kv_append_paged(k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                         lens.data_ptr(), block_table.data_ptr(), b, g, d_k, d_v, bs, mb, nb,
                                         int(max_len), _dtype_code(k_pool), _stream_handle(stream))
    _lib.check(rc, "gqa_kv_append_paged")


def decode_attention_paged(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           lens: torch.Tensor, block_table: torch.Tensor, max_len: int, scale: float,
                           workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Attention of q [b, h, d_k] over paged caches (pools [num_blocks, g, B, d], table [b, max_blocks])."""
    b, g, d_k, d_v, bs, mb, nb = _paged_args(k_pool, v_pool, block_table, lens)
    _check_gpu(k_pool, out, q, workspace)
    h = q.shape[1]
    if tuple(q.shape) != (b, h, d_k) or tuple(out.shape) != (b, h, d_v):
        raise ValueError("decode_attention_paged: q [b, h, d_k] and out [b, h, d_v] expected")
    if any(_dtype_code(t) != _dtype_code(q) for t in (k_pool, v_pool, out)):
        raise TypeError("q, pools and out must share one element type")
    rc = _lib.load().gqa_decode_attention_paged(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), lens.data_ptr(), block_table.data_ptr(),
        b, h, g, d_k, d_v, bs, mb, nb, int(max_len), float(scale), _dtype_code(q), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check(rc, "gqa_decode_attention_paged")
    return out


def decode_step_paged(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      k_pool: torch.Tensor, v_pool: torch.Tensor, lens: torch.Tensor, block_table: torch.Tensor,
                      max_len: int, scale: float, workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Append + attention in one launch on paged caches (max_len: bound of the pre-append lengths)."""
    b, g, d_k, d_v, bs, mb, nb = _paged_args(k_pool, v_pool, block_table, lens)
    _check_gpu(k_pool, out, q, k_new, v_new, workspace)
    h = q.shape[1]
    if tuple(q.shape) != (b, h, d_k) or tuple(out.shape) != (b, h, d_v) or tuple(k_new.shape) != (b, g, d_k) \
            or tuple(v_new.shape) != (b, g, d_v):
        raise ValueError("decode_step_paged: inconsistent shapes")
    if any(_dtype_code(t) != _dtype_code(q) for t in (k_pool, v_pool, out, k_new, v_new)):
        raise TypeError("q, rows, pools and out must share one element type")
    rc = _lib.load().gqa_decode_step_paged(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        lens.data_ptr(), block_table.data_ptr(), b, h, g, d_k, d_v, bs, mb, nb, int(max_len), float(scale),
        _dtype_code(q), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check(rc, "gqa_decode_step_paged")
    return out


def make_multi_workspace(b: int, n: int, h: int, g: int, d_k: int, d_v: int, dtype: torch.dtype, device):
    """Zeroed workspace for the multi-token calls (gqa_decode_multi_workspace_size bytes)."""
    nbytes = int(_lib.load().gqa_decode_multi_workspace_size(b, n, h, g, d_k, d_v, _DTYPES[dtype]))
    if nbytes == 0:
        raise ValueError("unsupported shape for the multi-token workspace")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _multi_shapes(q, k_cache, v_cache, lens):
    _check_gpu(q, k_cache, v_cache, lens)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    b, n, h, d_k = q.shape
    bk, g, cap, dk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if bk != b or dk2 != d_k or tuple(v_cache.shape) != (b, g, cap, d_v) or tuple(lens.shape) != (b,):
        raise ValueError("multi-token call: inconsistent shapes")
    return b, n, h, g, cap, d_k, d_v


def kv_append_multi(k_cache, v_cache, k_new, v_new, lens, max_len: int, stream=None) -> None:
    """Store token r's rows (k_new / v_new [b, n, g, d]) at position lens[s] + r; lens += n."""
    _check_gpu(k_cache, v_cache, k_new, v_new, lens)
    b, n, g, d_k = k_new.shape
    if tuple(k_cache.shape[:2]) != (b, g) or tuple(v_new.shape[:3]) != (b, n, g) or lens.dtype != torch.int32 \
            or tuple(lens.shape) != (b,) or k_cache.shape[3] != d_k or v_cache.shape[3] != v_new.shape[3] \
            or tuple(v_cache.shape[:3]) != tuple(k_cache.shape[:3]):
        raise ValueError("kv_append_multi: inconsistent shapes")
    dt = _dtype_code(k_cache)
    if any(_dtype_code(t) != dt for t in (v_cache, k_new, v_new)):
        raise TypeError("caches and new rows must share one element type")
    rc = _lib.load().gqa_kv_append_multi(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                         lens.data_ptr(), b, n, g, d_k, v_cache.shape[3], k_cache.shape[2],
                                         int(max_len), dt, _stream_handle(stream))
    _lib.check(rc, "gqa_kv_append_multi")


def decode_attention_multi(out, q, k_cache, v_cache, lens, max_len: int, scale: float, workspace,
                           stream=None) -> torch.Tensor:
    """n query tokens per sequence (q, out [b, n, h, d]) over caches that already hold them, causal."""
    b, n, h, g, cap, d_k, d_v = _multi_shapes(q, k_cache, v_cache, lens)
    _check_gpu(out, workspace)
    if tuple(out.shape) != (b, n, h, d_v):
        raise ValueError("decode_attention_multi: out must be [b, n, h, d_v]")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_cache, v_cache, out)):
        raise TypeError("q, caches and out must share one element type")
    rc = _lib.load().gqa_decode_attention_multi(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(), b, n, h, g, d_k, d_v,
        cap, int(max_len), float(scale), dt, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_handle(stream))
    _lib.check(rc, "gqa_decode_attention_multi")
    return out


def decode_step_multi(out, q, k_new, v_new, k_cache, v_cache, lens, max_len: int, scale: float, workspace,
                      stream=None) -> torch.Tensor:
    """Append n tokens per sequence, then their causal attention (max_len: bound before the append)."""
    b, n, h, g, cap, d_k, d_v = _multi_shapes(q, k_cache, v_cache, lens)
    _check_gpu(out, k_new, v_new, workspace)
    if tuple(out.shape) != (b, n, h, d_v) or tuple(k_new.shape) != (b, n, g, d_k) \
            or tuple(v_new.shape) != (b, n, g, d_v):
        raise ValueError("decode_step_multi: inconsistent shapes")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_cache, v_cache, out, k_new, v_new)):
        raise TypeError("q, rows, caches and out must share one element type")
    rc = _lib.load().gqa_decode_step_multi(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        lens.data_ptr(), b, n, h, g, d_k, d_v, cap, int(max_len), float(scale), dt, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check(rc, "gqa_decode_step_multi")
    return out


def kv_append_multi_paged(k_pool, v_pool, k_new, v_new, lens, block_table, max_len: int, stream=None) -> None:
    """Store token r's rows (k_new / v_new [b, n, g, d]) at position lens[s] + r of each paged cache; lens += n."""
    b, g, d_k, d_v, bs, mb, nb = _paged_args(k_pool, v_pool, block_table, lens)
    _check_gpu(k_new, v_new)
    n = k_new.shape[1] if k_new.dim() == 4 else 0
    if tuple(k_new.shape) != (b, n, g, d_k) or tuple(v_new.shape) != (b, n, g, d_v):
        raise ValueError("kv_append_multi_paged: k_new [b, n, g, d_k] and v_new [b, n, g, d_v] expected")
    dt = _dtype_code(k_pool)
    if any(_dtype_code(t) != dt for t in (v_pool, k_new, v_new)):
        raise TypeError("pools and new rows must share one element type")
    rc = _lib.load().gqa_kv_append_multi_paged(
        k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), lens.data_ptr(),
        block_table.data_ptr(), b, n, g, d_k, d_v, bs, mb, nb, int(max_len), dt, _stream_handle(stream))
    _lib.check(rc, "gqa_kv_append_multi_paged")


def _multi_paged_shapes(out, q, k_pool, v_pool, lens, block_table):
    b, g, d_k, d_v, bs, mb, nb = _paged_args(k_pool, v_pool, block_table, lens)
    _check_gpu(out, q)
    if q.dim() != 4:
        raise ValueError("q must be [b, n, h, d_k]")
    n, h = q.shape[1], q.shape[2]
    if tuple(q.shape) != (b, n, h, d_k) or tuple(out.shape) != (b, n, h, d_v):
        raise ValueError("multi-token paged call: q [b, n, h, d_k] and out [b, n, h, d_v] expected")
    return b, n, h, g, d_k, d_v, bs, mb, nb


def decode_attention_multi_paged(out, q, k_pool, v_pool, lens, block_table, max_len: int, scale: float, workspace,
                                 stream=None) -> torch.Tensor:
    """n query tokens per sequence (q, out [b, n, h, d]) over paged caches that already hold them, causal."""
    b, n, h, g, d_k, d_v, bs, mb, nb = _multi_paged_shapes(out, q, k_pool, v_pool, lens, block_table)
    _check_gpu(workspace)
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_pool, v_pool, out)):
        raise TypeError("q, pools and out must share one element type")
    rc = _lib.load().gqa_decode_attention_multi_paged(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), lens.data_ptr(), block_table.data_ptr(),
        b, n, h, g, d_k, d_v, bs, mb, nb, int(max_len), float(scale), dt, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check(rc, "gqa_decode_attention_multi_paged")
    return out


def decode_step_multi_paged(out, q, k_new, v_new, k_pool, v_pool, lens, block_table, max_len: int, scale: float,
                            workspace, stream=None) -> torch.Tensor:
    """Append n tokens per sequence to paged caches, then their causal attention (max_len: bound before)."""
    b, n, h, g, d_k, d_v, bs, mb, nb = _multi_paged_shapes(out, q, k_pool, v_pool, lens, block_table)
    _check_gpu(k_new, v_new, workspace)
    if tuple(k_new.shape) != (b, n, g, d_k) or tuple(v_new.shape) != (b, n, g, d_v):
        raise ValueError("decode_step_multi_paged: k_new [b, n, g, d_k] and v_new [b, n, g, d_v] expected")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k_pool, v_pool, out, k_new, v_new)):
        raise TypeError("q, rows, pools and out must share one element type")
    rc = _lib.load().gqa_decode_step_multi_paged(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        lens.data_ptr(), block_table.data_ptr(), b, n, h, g, d_k, d_v, bs, mb, nb, int(max_len), float(scale), dt,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check(rc, "gqa_decode_step_multi_paged")
    return out
