"""Seeded generators for the decode workloads (no method arithmetic here).

Every random quantity is drawn from its own NumPy PCG64 stream, keyed by a
``SeedSequence`` spawn key, so any piece of any workload can be regenerated on
its own (a sampled parity check regenerates only the requests it needs):

=============================  ==========================================
stream (spawn key)             contents
=============================  ==========================================
``(0, b)``                     Q of request ``b``: fp32 N(0, 1), ``[Sq, H, 576]``
``(1, b, k)``                  KV tokens ``[k*65536, (k+1)*65536)`` of request
                               ``b`` in logical order: fp32 N(0, 1), 576 wide
``(2, b, k)``                  outlier mask for the same KV chunk (Bernoulli)
``(3,)``                       per-request context lengths, uniform integers
``(4,)``                       permutation of the shared page pool
=============================  ==========================================

The KV row is 576 wide: 512 latent columns followed by 64 rope columns, and the
value vector is the first 512 columns of the same row.  These shapes, the
N(0, 1) values, the 1 % x1000 outliers, the U[4096, 131072] lengths, the
page size of 64 and the permuted shared pool describe synthetic stand-ins for
the long-context decode workloads (batch 1 and 16 at 128K context, a paged
batch of 32, and an 8-token speculative verify at 1M context); no dataset or
trained weights are involved.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

D_KV = 576          # latent 512 + rope 64
D_V = 512           # value = first 512 columns of the KV row
D_ROPE = D_KV - D_V
CHUNK_TOKENS = 65536


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one decode workload."""

    name: str
    batch: int
    heads: int
    q_tokens: int                     # Sq: query tokens per request (causal among them)
    context: Optional[int]            # fixed context length per request, or None
    context_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    page_size: int = 0                # 0: contiguous per-request KV
    permuted_pool: bool = False
    outlier_frac: float = 0.0         # fraction of KV source values multiplied
    outlier_mult: float = 1.0
    num_splits: Optional[int] = None  # None: chosen by the split planner
    seed: int = 0
    softmax_scale: float = 1.0 / math.sqrt(192.0)

    @property
    def rows(self) -> int:
        return self.q_tokens * self.heads


WORKLOADS = {
    "tiny": Workload("tiny_b1_h16_l256", batch=1, heads=16, q_tokens=1, context=256,
                     num_splits=4),
    "b1_128k": Workload("b1_h128_l131072", batch=1, heads=128, q_tokens=1, context=131072,
                        num_splits=64),
    "b16_128k": Workload("b16_h128_l131072_contig", batch=16, heads=128, q_tokens=1,
                         context=131072),
    "paged_b32": Workload("paged_b32_h128_p64_u4k_128k", batch=32, heads=128, q_tokens=1,
                          context=None, context_range=(4096, 131072), page_size=64,
                          permuted_pool=True, outlier_frac=0.01, outlier_mult=1000.0),
    "verify_b4_1m": Workload("verify_b4_h128_sq8_l1048576", batch=4, heads=128, q_tokens=8,
                             context=1048576),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed,
                                                                       spawn_key=tuple(key))))


def seq_lens_for(w: Workload) -> np.ndarray:
    """Per-request context lengths (they include the Sq new query tokens)."""
    if w.context is not None:
        return np.full(w.batch, w.context, dtype=np.int32)
    lo, hi = w.context_range
    return _rng(w.seed, 3).integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)


def q_f32(w: Workload, b: Optional[int] = None) -> np.ndarray:
    """Q as fp32 N(0,1): ``[B, Sq, H, 576]`` (or ``[Sq, H, 576]`` for one request)."""
    if b is not None:
        return _rng(w.seed, 0, b).standard_normal((w.q_tokens, w.heads, D_KV), dtype=np.float32)
    return np.stack([q_f32(w, i) for i in range(w.batch)])


def kv_chunk_f32(w: Workload, b: int, k: int, length: int) -> np.ndarray:
    """KV rows ``[k*CHUNK, k*CHUNK+length)`` of request ``b``: fp32 N(0,1), 576 wide.

    Values are drawn row-major from the chunk's own stream, so a shorter draw
    is a prefix of a longer one.
    """
    assert 0 <= length <= CHUNK_TOKENS
    return _rng(w.seed, 1, b, k).standard_normal((length, D_KV), dtype=np.float32)


def outlier_mask(w: Workload, b: int, k: int, length: int) -> np.ndarray:
    """Boolean mask of the source values that get multiplied by ``outlier_mult``."""
    if w.outlier_frac <= 0.0:
        return np.zeros((length, D_KV), dtype=bool)
    return _rng(w.seed, 2, b, k).random((length, D_KV), dtype=np.float32) < w.outlier_frac


def kv_request_f32(w: Workload, b: int, seq_len: int, with_outliers: bool = True,
                   threads: Optional[int] = None) -> np.ndarray:
    """All KV rows of request ``b`` in logical order, ``[seq_len, 576]`` fp32.

    With ``with_outliers`` the masked source values are multiplied by
    ``outlier_mult`` (this is part of the input recipe, not of the method).
    """
    n_chunks = (seq_len + CHUNK_TOKENS - 1) // CHUNK_TOKENS
    out = np.empty((seq_len, D_KV), dtype=np.float32)

    def fill(k: int) -> None:
        lo = k * CHUNK_TOKENS
        n = min(CHUNK_TOKENS, seq_len - lo)
        x = kv_chunk_f32(w, b, k, n)
        if with_outliers and w.outlier_frac > 0.0:
            x[outlier_mask(w, b, k, n)] *= np.float32(w.outlier_mult)
        out[lo:lo + n] = x

    nt = threads or min(16, len(os.sched_getaffinity(0)))
    if n_chunks <= 1 or nt <= 1:
        for k in range(n_chunks):
            fill(k)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def page_layout(w: Workload, seq_lens: np.ndarray):
    """Page size, page table ``[B, max_pages]`` int32 and pool page count.

    Paged workloads use a shared pool holding exactly sum(ceil(L_b / P)) pages,
    handed out in a random permutation; unused table entries are 0.  Contiguous
    workloads use one page per request, sized ceil(max L / 64) * 64 tokens.
    """
    if w.page_size == 0:
        p = int(-(-int(seq_lens.max()) // 64) * 64)
        table = np.arange(w.batch, dtype=np.int32).reshape(w.batch, 1)
        return p, table, w.batch
    p = w.page_size
    n_pages = [(-(-int(L) // p)) for L in seq_lens]
    total = int(sum(n_pages))
    order = np.arange(total, dtype=np.int64)
    if w.permuted_pool:
        order = _rng(w.seed, 4).permutation(total)
    table = np.zeros((w.batch, max(n_pages)), dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = order[off:off + n]
        off += n
    return p, table, total
