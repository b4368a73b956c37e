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

A third piece, from the theainews.cc page on Muse Spark Open, section "内核优化:解码吞吐 3 倍",
item "RoPE 与 KV 缓存写入融合" (rotary position embedding fused with the KV-cache write): the
append may rotate the rope part of each new row before it is quantised.  Readings:

* the 64 rope columns (512 .. 575) form 32 pairs of adjacent columns (512 + 2i, 513 + 2i),
  each a complex number x0 + i x1 multiplied by cos + i sin of its angle;
* the angles come from the caller as tables cos[position, 32] and sin[position, 32]
  (fp32), so no model's frequency schedule is built in; position n = seq_lens[b] - T + t;
* the rotation is computed in fp32 with every product and sum rounded on its own
  (r0 = fl(fl(x0 c) - fl(x1 s)), r1 = fl(fl(x0 s) + fl(x1 c))), because the rounding of
  the rotated value decides its E4M3 code; the latent columns are not touched;
* a position at or past the end of the tables is not written (as a position past the
  page table).

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


def rope_rotate_f32(row, cos_row, sin_row) -> np.ndarray:
    """A 576-wide fp32 row with its rope pairs (512 + 2i, 513 + 2i) rotated by (cos_row[i],
    sin_row[i]), every product and sum rounded to fp32 on its own; latent columns unchanged."""
    x = np.array(row, dtype=np.float32, copy=True)
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    x0, x1 = x[512::2].copy(), x[513::2].copy()
    x[512::2] = (x0 * c).astype(np.float32) - (x1 * s).astype(np.float32)
    x[513::2] = (x0 * s).astype(np.float32) + (x1 * c).astype(np.float32)
    return x


def append_kv_rope_fp8(kv_pool8: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray,
                       new_kv, kv_scale, cos_table, sin_table) -> np.ndarray:
    """append_kv_fp8 with each new row's rope part rotated first by the angle of its position
    (cos_table / sin_table: fp32 [positions, 32]); positions past the tables are not written."""
    pool = np.array(kv_pool8, dtype=np.uint8, copy=True)
    num_pages, page_size, _ = pool.shape
    new_kv = np.asarray(new_kv, dtype=np.float32)
    batch, t_new, _ = new_kv.shape
    max_pages = page_table.shape[1]
    n_pos = cos_table.shape[0]
    for b in range(batch):
        for t in range(t_new):
            n = int(seq_lens[b]) - t_new + t
            if n < 0 or n >= max_pages * page_size or n >= n_pos:
                continue
            page = int(page_table[b, n // page_size])
            if page < 0 or page >= num_pages:
                continue
            row = rope_rotate_f32(new_kv[b, t], cos_table[n], sin_table[n])
            pool[page, n % page_size] = quantize_e4m3_sat(row, kv_scale)
    return pool
