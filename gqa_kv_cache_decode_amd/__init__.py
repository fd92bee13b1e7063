"""MI355X-native incremental decoding attention for MHA / GQA / MQA.

One decode step appends one token of K/V per sequence to its cache and then
lets that token's h query heads attend over the whole cache, sharing g KV
heads (g = h is MHA, g = 1 is MQA). The work is done by hand-written HIP
kernels for gfx950 behind the C ABI in ``include/gqa_decode.h``; this package
is the thin Python binding over that library (``api``), plus the seeded
synthetic inputs (``inputs``) and workload table (``workloads``).

Importing the package loads nothing native; the library is loaded on the
first call and a missing library is an error, never a fallback.
"""
__version__ = "0.1.0"

__all__ = ["api", "inputs", "workloads"]
