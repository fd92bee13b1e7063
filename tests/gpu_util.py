"""Helpers shared by the GPU tests: host <-> device copies and the parity bar.

Parity bar for decode outputs (compared against the fp64 oracle):
* fp32 inputs: max |gpu - oracle| <= 1e-5;
* bf16 inputs (fp32 accumulation, bf16 output): max |gpu - oracle| <= 2e-2
  and, for every (sequence, head) row, ||gpu - oracle||_2 / ||oracle||_2
  <= 1e-2 (an elementwise relative bound is ill-posed for outputs that cross
  zero, and the absolute bound alone is loose at long lengths where outputs
  are small).
Cache appends are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

from gqa_kv_cache_decode_amd import inputs

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_ROW_REL = 1e-2


def to_dev(arr: np.ndarray, device="cuda") -> torch.Tensor:
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the oracle's storage type (float32 or bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def to_f64(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return inputs.bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def parity_report(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    num = np.sqrt(((got - ref) ** 2).sum(axis=-1))
    den = np.sqrt((ref ** 2).sum(axis=-1))
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    return {"max_abs": float(err.max(initial=0.0)), "max_row_rel": float(rel.max(initial=0.0)),
            "finite": bool(np.isfinite(got).all())}


def assert_parity(got_dev: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    got = to_f64(to_host_bits(got_dev))
    rep = parity_report(got, ref)
    assert rep["finite"], f"{what}: non-finite GPU output"
    if dtype == "f32":
        assert rep["max_abs"] <= F32_MAX_ABS, f"{what}: {rep}"
    else:
        assert rep["max_abs"] <= BF16_MAX_ABS, f"{what}: {rep}"
        assert rep["max_row_rel"] <= BF16_ROW_REL, f"{what}: {rep}"
    return rep


STAMP_BYTES = 65792  # the workspace's last bytes: spread-merge stamps, never reset


def counter_bytes(ws, b, h):
    """The workspace's counter region (36864 + c bytes before its last 65792, as the header states)."""
    bh = b * h
    n = 32 * bh if bh <= 8192 else max(bh, 262144)
    usable = (ws.numel() * ws.element_size()) & ~255
    cnt = ((4 * n + 255) // 256) * 256
    return ws.view(torch.uint8)[usable - STAMP_BYTES - 36864 - cnt: usable - STAMP_BYTES]


def stamp_words(ws):
    """The spread merge's generation words (launch generation, generation whose workgroups all started)."""
    usable = (ws.numel() * ws.element_size()) & ~255
    words = ws.view(torch.uint8)[usable - STAMP_BYTES: usable - STAMP_BYTES + 256].view(torch.int32)
    return int(words[0]), int(words[32])


def assert_counters_zero(ws, b, h):
    region = counter_bytes(ws, b, h)
    assert int(region.view(torch.int32).abs().sum()) == 0, "workspace counters not back to zero"
