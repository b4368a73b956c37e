"""Seeded synthetic inputs for the FP8 MLA split-KV decode workloads.

This package only draws random numbers and lays them out.  It holds none of
the method's arithmetic: no quantisation, no scale computation, no attention.
Both the CPU oracle (``oracle/``) and the GPU path's tests and benchmark take
their inputs from here, so the two sides see the same fp32 values.
"""
from .gen import (  # noqa: F401
    CHUNK_TOKENS,
    D_KV,
    D_V,
    WORKLOADS,
    Workload,
    kv_request_f32,
    kv_chunk_f32,
    outlier_mask,
    page_layout,
    q_f32,
    seq_lens_for,
)
