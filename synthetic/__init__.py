"""Seeded synthetic inputs for the DSA hot path, shared by tests, smoke and bench.

This package holds none of the method's arithmetic: only random draws, the
round-to-nearest-even cast of fp32 draws to bfloat16, and the FP8 block
quantisation that produces a stored FP8 key cache (the stored format the
indexer consumes).  Every element is a pure function of
(seed, tensor id, leading index), so any single sequence of a large workload
can be regenerated on its own.
"""
from .gen import (  # noqa: F401
    causal_index_lists,
    normal,
    page_table,
    quantize_fp8_blocks,
    scatter_pages,
    uniform_int,
)
from .workloads import WORKLOADS, make_workload  # noqa: F401
