"""The decode workloads this library is checked and measured on.

Each entry fixes the problem shape, the element type, the pre-append cache
lengths, the capacity (room for every appended token) and the seed of the
input generator. Model names describe shapes only; no weights are involved.

* ``tiny_gqa_f32``: b=2, h=4, g=2, d=16, fp32, lengths 37 and 64.
* ``mqa_bf16``: b=8, h=32, g=1, d=128, bf16, length 4096.
* ``llama3_70b_gqa_bf16``: one Llama-3-70B-shaped layer, b=16, h=64, g=8,
  d=128, bf16, lengths uniform on [1024, 8192].
* ``qwen25_7b_gqa_bf16``: Qwen2.5-7B-shaped, b=64, h=28, g=4, d=128, bf16,
  length 2048 growing to 2080 over a 32-step decode loop.
* ``mha_long_bf16_g{32,8,1}``: b=4, h=32, d=128, bf16, length 32768, at g=32
  (MHA), g=8 and g=1 (MQA) from the same seed, to show bytes read scale with g.

Scale is 1/sqrt(d) rounded to fp32 for all of them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    h: int
    g: int
    d: int
    dtype: str
    lens: object  # int, list of ints, or ("uniform", lo, hi)
    cap: int
    seed: int
    steps: int = 1
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        import numpy as np
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_gqa_f32", b=2, h=4, g=2, d=16, dtype="f32", lens=[37, 64], cap=128, seed=1001),
        Workload("mqa_bf16", b=8, h=32, g=1, d=128, dtype="bf16", lens=4096, cap=4160, seed=1002),
        Workload("llama3_70b_gqa_bf16", b=16, h=64, g=8, d=128, dtype="bf16",
                 lens=("uniform", 1024, 8192), cap=8256, seed=1003),
        Workload("qwen25_7b_gqa_bf16", b=64, h=28, g=4, d=128, dtype="bf16", lens=2048, cap=2112,
                 seed=1004, steps=32),
        Workload("mha_long_bf16_g32", b=4, h=32, g=32, d=128, dtype="bf16", lens=32768, cap=32832, seed=1005),
        Workload("mha_long_bf16_g8", b=4, h=32, g=8, d=128, dtype="bf16", lens=32768, cap=32832, seed=1005),
        Workload("mha_long_bf16_g1", b=4, h=32, g=1, d=128, dtype="bf16", lens=32768, cap=32832, seed=1005),
    ]
}

HEADLINE = "llama3_70b_gqa_bf16"


def kv_bytes_attended(g: int, d_k: int, d_v: int, elem_bytes: int, attended_lens) -> int:
    """Bytes of K and V one attention pass must read: sum_b g * L_b * (d_k + d_v) * e."""
    return int(sum(int(x) for x in attended_lens)) * g * (d_k + d_v) * elem_bytes
