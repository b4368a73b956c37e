"""Materialise a synthetic decode workload in device memory through the library.

The seeded fp32 values come from ``synthetic``; everything computed from them runs in the
library's kernels.  Q is quantised by ``mla_quantize_fp8_sat_dynamic``, whose per-tensor
scale (max|x| / 448) is taken from the data on the GPU.  The KV scale is taken the same way
over all requests' values at once (for the outlier workload over the values before the x1000
injection, so that 1 % of the values saturate), and every request's rows are then converted
by ``mla_quantize_fp8_sat`` with it.  Pages of a paged workload are placed in the shared
pool through the page table; rows of a page past the end of its request hold 0x7F (NaN)
bytes, so any read of them would poison the result.  The scales are read back once as host
floats for the calls that take them by value.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from synthetic import D_KV, Workload, kv_request_f32, page_layout, q_f32, seq_lens_for

from .mla import quantize_fp8_sat, quantize_fp8_sat_dynamic

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
    kv_f32: Optional[List[torch.Tensor]] = None  # per request, device fp32 (if kept)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens_host.max())

    @property
    def kv_tokens(self) -> int:
        return int(self.seq_lens_host.sum())


def materialize(w: Workload, device: str = "cuda", keep_f32: bool = False,
                seq_lens: Optional[np.ndarray] = None) -> DeviceWorkload:
    """Build the workload on ``device``.  ``seq_lens`` overrides the recipe's lengths."""
    lens = seq_lens_for(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    P, table, n_pages = page_layout(w, lens)

    q8, q_scale_dev = quantize_fp8_sat_dynamic(torch.from_numpy(q_f32(w)).to(device))

    # every request's fp32 rows in one device tensor, so that one call takes the scale over all
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))])
    total = int(offs[-1])
    kv_all = torch.empty((max(total, 1), D_KV), dtype=torch.float32, device=device)
    for b, L in enumerate(lens):
        if L > 0:
            kv_all[offs[b]:offs[b + 1]] = torch.from_numpy(
                kv_request_f32(w, b, int(L), with_outliers=False)).to(device)
    kv_scale = 1.0
    if total > 0:
        codes, kv_scale_dev = quantize_fp8_sat_dynamic(kv_all[:total])
        del codes
        kv_scale = float(kv_scale_dev.item())
    if w.outlier_frac > 0.0:
        for b, L in enumerate(lens):
            if L > 0:
                kv_all[offs[b]:offs[b + 1]] = torch.from_numpy(
                    kv_request_f32(w, b, int(L), with_outliers=True)).to(device)

    pool = torch.full((n_pages, P, D_KV), NAN_BYTE, dtype=torch.uint8, device=device)
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        n = -(-L // P)
        staged = torch.full((n * P, D_KV), NAN_BYTE, dtype=torch.uint8, device=device)
        quantize_fp8_sat(kv_all[offs[b]:offs[b + 1]], kv_scale, out=staged[:L])
        idx = torch.from_numpy(table[b, :n].astype(np.int64)).to(device)
        pool.index_copy_(0, idx, staged.view(n, P, D_KV))
        del staged
    kv_f32 = None
    if keep_f32:
        kv_f32 = [kv_all[offs[b]:offs[b + 1]] for b in range(len(lens))]
    else:
        del kv_all
    torch.cuda.synchronize(device)
    return DeviceWorkload(
        w=w, q8=q8, kv_pool8=pool,
        page_table=torch.from_numpy(table).to(device),
        seq_lens=torch.from_numpy(lens).to(device),
        seq_lens_host=lens, page_table_host=table, page_size=P,
        q_scale=float(q_scale_dev.item()), kv_scale=kv_scale, kv_f32=kv_f32)
