"""Materialise a synthetic decode workload in device memory.

Host side: the seeded fp32 values come from ``synthetic`` and the per-tensor scales are
max|x| / 448 in fp32 (for the outlier workload the KV scale uses the values before the x1000
injection, so 1 % of the values saturate).  Device side: the fp32 values are uploaded and
converted to E4M3 by ``mla_quantize_fp8_sat``; pages of a paged workload are then placed in
the shared pool through the page table.  Rows of a page past the end of its request hold
0x7F (NaN) bytes, so any read of them would poison the result.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from synthetic import D_KV, Workload, kv_request_f32, page_layout, q_f32, seq_lens_for

from .mla import quantize_fp8_sat

NAN_BYTE = 0x7F


@dataclass
class DeviceWorkload:
    w: Workload
    q8: torch.Tensor            # [B, Sq, H, 576] uint8
    kv_pool8: torch.Tensor      # [pages, P, 576] uint8
    page_table: torch.Tensor    # [B, max_pages] int32 (device)
    seq_lens: torch.Tensor      # [B] int32 (device)
    seq_lens_host: np.ndarray
    page_table_host: np.ndarray
    page_size: int
    q_scale: float
    kv_scale: float
    q_amax: float
    kv_amax: float
    kv_f32: Optional[List[torch.Tensor]] = None  # per request, device fp32 (if kept)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens_host.max())

    @property
    def kv_tokens(self) -> int:
        return int(self.seq_lens_host.sum())


def _scale(amax: float) -> float:
    a = np.float32(amax)
    return float(a / np.float32(448.0)) if a > 0 else 1.0


def materialize(w: Workload, device: str = "cuda", keep_f32: bool = False,
                seq_lens: Optional[np.ndarray] = None) -> DeviceWorkload:
    """Build the workload on ``device``.  ``seq_lens`` overrides the recipe's lengths."""
    lens = seq_lens_for(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    P, table, n_pages = page_layout(w, lens)

    q = q_f32(w)
    q_amax = float(np.abs(q).max())
    q_scale = _scale(q_amax)
    q8 = quantize_fp8_sat(torch.from_numpy(q).to(device), q_scale)

    kv_dev, amax = [], 0.0
    for b, L in enumerate(lens):
        base = kv_request_f32(w, b, int(L), with_outliers=False)
        amax = max(amax, float(np.abs(base).max())) if L > 0 else amax
        if w.outlier_frac > 0.0:
            base = kv_request_f32(w, b, int(L), with_outliers=True)
        kv_dev.append(torch.from_numpy(base).to(device))
        del base
    kv_scale = _scale(amax)

    pool = torch.full((n_pages, P, D_KV), NAN_BYTE, dtype=torch.uint8, device=device)
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        n = -(-L // P)
        staged = torch.full((n * P, D_KV), NAN_BYTE, dtype=torch.uint8, device=device)
        quantize_fp8_sat(kv_dev[b], kv_scale, out=staged[:L])
        idx = torch.from_numpy(table[b, :n].astype(np.int64)).to(device)
        pool.index_copy_(0, idx, staged.view(n, P, D_KV))
        del staged
    torch.cuda.synchronize(device)
    return DeviceWorkload(
        w=w, q8=q8, kv_pool8=pool,
        page_table=torch.from_numpy(table).to(device),
        seq_lens=torch.from_numpy(lens).to(device),
        seq_lens_host=lens, page_table_host=table, page_size=P,
        q_scale=q_scale, kv_scale=kv_scale, q_amax=q_amax, kv_amax=amax,
        kv_f32=kv_dev if keep_f32 else None)
