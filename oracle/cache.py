"""Preparing the FP8 KV cache and Q for a decode step, from the definitions.

[A/MLA] item (4): Q and KV are converted to FP8 with a saturating cast before the
attention reads them.  Two pieces of that preparation are stated here:

* appending a step's new latent + rope rows to a paged FP8 cache: each new row is
  quantised with the cache's scale and stored where the attention will look for it;
* a per-tensor scale taken from the data itself (amax / 448, as ``per_tensor_scale``)
  for a tensor that arrives as fp32 or as bf16.

Readings (the pages give neither layout nor interface):

* ``seq_lens[b]`` already counts the T new tokens (the same convention the attention
  uses), so new token t of request b is logical position n = seq_lens[b] - T + t;
* logical position n lives in row n % P of pool page ``page_table[b, n // P]``;
* a position outside [0, max_pages * P), or a page id outside the pool, is not
  written (nothing else in the pool changes);
* bf16 is the upper half of an IEEE fp32 bit pattern, so its value is exactly the
  fp32 whose low 16 bits are zero; the scale and quotients are then those of fp32.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import per_tensor_scale, quantize_e4m3_sat

D_KV = 576


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Values of bf16 bit patterns (uint16) as float32: the pattern is the fp32's upper half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def dynamic_quantize(x, source: str = "f32"):
    """Per-tensor scale from the data, then the saturating encode: ``(codes, scale)``.

    ``source`` is "f32" (x holds float32 values) or "bf16" (x holds bf16 bit patterns)."""
    xf = bf16_bits_to_f32(x) if source == "bf16" else np.asarray(x, dtype=np.float32)
    s = per_tensor_scale(xf)
    return quantize_e4m3_sat(xf, s), s


def append_kv_fp8(kv_pool8: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray,
                  new_kv, kv_scale) -> np.ndarray:
    """A copy of ``kv_pool8`` [pages, P, 576] with the rows of ``new_kv`` [B, T, 576] (fp32)
    quantised with ``kv_scale`` and written at their logical positions."""
    pool = np.array(kv_pool8, dtype=np.uint8, copy=True)
    num_pages, page_size, _ = pool.shape
    new_kv = np.asarray(new_kv, dtype=np.float32)
    batch, t_new, _ = new_kv.shape
    max_pages = page_table.shape[1]
    for b in range(batch):
        for t in range(t_new):
            n = int(seq_lens[b]) - t_new + t
            if n < 0 or n >= max_pages * page_size:
                continue
            page = int(page_table[b, n // page_size])
            if page < 0 or page >= num_pages:
                continue
            pool[page, n % page_size] = quantize_e4m3_sat(new_kv[b, t], kv_scale)
    return pool
