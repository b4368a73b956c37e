"""Oracle side of the GPU parity tests: regenerate inputs on the host and run ``oracle/``.

Nothing here reads a GPU result.  Large workloads are handled per 65,536-token chunk of the
synthetic generator; each chunk is regenerated and quantised by the oracle in a worker
process (the pool forks from a server started before any GPU use, see conftest.py).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
from typing import Optional, Sequence

import numpy as np

from oracle import attention_fp64, per_tensor_scale, quantize_e4m3_sat
from synthetic import CHUNK_TOKENS, D_KV, Workload, kv_chunk_f32, outlier_mask, q_f32

_POOL = None


def pool() -> Optional[ProcessPoolExecutor]:
    global _POOL
    if _POOL is None:
        import multiprocessing as mp
        n = min(16, len(os.sched_getaffinity(0)))
        if n > 1:
            _POOL = ProcessPoolExecutor(n, mp_context=mp.get_context("forkserver"))
    return _POOL


def _chunk_amax(args):
    w, b, k, n = args
    return float(np.abs(kv_chunk_f32(w, b, k, n)).max()) if n else 0.0


def _chunk_codes(args):
    w, b, k, n, scale = args
    x = kv_chunk_f32(w, b, k, n)
    if w.outlier_frac > 0.0:
        x[outlier_mask(w, b, k, n)] *= np.float32(w.outlier_mult)
    return quantize_e4m3_sat(x, scale)


def _chunks(w: Workload, b: int, L: int):
    return [(w, b, k, min(CHUNK_TOKENS, L - k * CHUNK_TOKENS))
            for k in range(-(-L // CHUNK_TOKENS))]


def _map(fn, items):
    p = pool()
    return list(p.map(fn, items)) if p is not None and len(items) > 1 else [fn(i) for i in items]


def scales(w: Workload, lens: Sequence[int]):
    """Oracle per-tensor scales: Q over all of Q; KV over every request's values before the
    outlier injection (the static calibrated scale of the outlier workload)."""
    q_scale = per_tensor_scale(q_f32(w))
    items = [c for b, L in enumerate(lens) for c in _chunks(w, b, int(L))]
    amax = max(_map(_chunk_amax, items)) if items else 0.0
    return q_scale, per_tensor_scale(np.array([amax], dtype=np.float32))


def kv8_request(w: Workload, b: int, L: int, kv_scale) -> np.ndarray:
    """Oracle e4m3 codes of request b's KV rows in logical order, [L, 576]."""
    parts = _map(_chunk_codes, [c + (kv_scale,) for c in _chunks(w, b, L)])
    return np.concatenate(parts) if parts else np.zeros((0, D_KV), np.uint8)


def q8_request(w: Workload, b: int, q_scale) -> np.ndarray:
    return quantize_e4m3_sat(q_f32(w, b), q_scale)


def attention_request(w: Workload, b: int, L: int, q8_b: np.ndarray, q_scale, kv8: np.ndarray,
                      kv_scale, heads: Optional[Sequence[int]] = None,
                      q_len: Optional[int] = None):
    """Oracle O [Sq, h, 512] and lse [Sq, h] of one request, through a one-page pool;
    q_len: the request's own number of query tokens (default: all Sq slots)."""
    P = max(32, -(-L // 32) * 32)
    pool_ = np.zeros((1, P, D_KV), np.uint8)
    pool_[0, :L] = kv8
    o, lse = attention_fp64(q8_b[None], q_scale, pool_, kv_scale, np.zeros((1, 1), np.int32),
                            np.array([L], np.int32), P, w.softmax_scale, heads=heads,
                            q_lens=None if q_len is None else [q_len])
    return o[0], lse[0]


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# lse: 1e-3 absolute (fp32 softmax sums over up to 1M terms) plus 2^-15 of the larger of
# |lse| and, where the caller gives it, the row's largest sum of |score terms|.  The scores
# come from FP8 matrix instructions whose internal accumulation of a 64-term dot product is
# not exact fp32: measured on MI355X with one key (lse = its score), the raw dot product of
# e4m3 codes is off by up to about 1e-5 of the sum of its terms' magnitudes (the usual
# floating-point bound for a dot product), so a score of 140 (natural log units) can be off
# by 1.5e-3, as can a moderate score made of large terms that cancel, while the output,
# which depends on score differences, is not.
LSE_ATOL, LSE_RTOL = 1e-3, 2.0 ** -15


def check_output(o_gpu: np.ndarray, o_ref: np.ndarray, lse_gpu=None, lse_ref=None,
                 max_abs: float = 1e-2, mean_rel: float = 2e-3, lse_terms=None):
    """Accuracy contract: max |err| <= 1e-2 and sum|err| / sum|ref| <= 2e-3 on the bf16
    output; lse within LSE_ATOL + LSE_RTOL * max(|lse|, lse_terms) (see above; lse_terms, if
    given, holds per row the largest softmax_scale * sum_i |q_i k_i| over its visible keys,
    natural log units).

    The max-abs bound is on the value before its rounding to bf16: the output is allowed half
    a bf16 ulp more, at the larger of |ref| and |out| (bf16 keeps 8 significant bits, so
    half an ulp of x = m 2^e, 0.5 <= m < 1, is 2^(e - 9); 0.0156 for 4 <= |x| < 8, where no
    bf16 value lies within 1e-2 of every real number)."""
    err = np.abs(o_gpu - o_ref)
    nl1 = float(err.sum() / max(np.abs(o_ref).sum(), 1e-300))
    assert np.all(np.isfinite(o_gpu)), "non-finite output"
    _, e = np.frexp(np.maximum(np.abs(o_ref), np.abs(o_gpu)))
    excess = err - (max_abs + np.ldexp(1.0, e - 9))
    mx = float(err.max()) if err.size else 0.0
    if err.size and float(excess.max()) > 0:
        at = np.unravel_index(int(np.argmax(excess)), err.shape)
        raise AssertionError(f"abs error {err[at]:.3e} > {max_abs} + half a bf16 ulp of "
                             f"{float(max(abs(o_ref[at]), abs(o_gpu[at]))):.4f} at {at}")
    assert nl1 <= mean_rel, f"normalised L1 error {nl1:.3e} > {mean_rel}"
    if lse_ref is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_gpu))
        if fin.any():
            d = np.where(fin, np.abs(np.where(fin, lse_gpu, 0.0) - np.where(fin, lse_ref, 0.0)),
                         0.0)
            mag = np.abs(np.where(fin, lse_ref, 0.0))
            if lse_terms is not None:
                mag = np.maximum(mag, np.asarray(lse_terms, dtype=np.float64))
            bound = LSE_ATOL + LSE_RTOL * mag
            if np.any(d > bound):
                at = np.unravel_index(int(np.argmax(d - bound)), d.shape)
                raise AssertionError(f"lse error {d[at]:.3e} > {bound[at]:.3e} at {at} "
                                     f"(ref {lse_ref[at]:.6f}, got {lse_gpu[at]:.6f})")
    return mx, nl1
