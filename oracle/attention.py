"""MLA decode attention over dequantised FP8 values, float64, from the definition.

What is computed ([A/MLA] intro and items (1)-(3); [B] section
"MLAアテンションのパイプライン深化"): for every request, query token and head,
softmax attention of the query over that request's latent KV cache, where the
cache row is 576 wide (512 latent + 64 rope columns, shared by all heads) and
the value vector is the row's first 512 columns.  Splitting the KV of one
request into chunks and merging the chunks' partial results ([A/MLA] items
(2) and (3)) is an exact re-association of the same sum, so the oracle is the
unsplit definition; ``split_partials_fp64`` / ``combine_fp64`` restate the
split form only so that tests can check the identity.

Readings (the pages give no formulas):

* scores z = softmax_scale * (q_scale * dec(Q8)) . (kv_scale * dec(K8)); the
  output is sum_n softmax(z)_n * V_n and lse = log(sum_n exp(z_n)) (natural log);
* ``seq_lens[b]`` counts the whole context including the Sq query tokens; the
  query tokens are the last Sq positions, so query token t (0-based) sees
  positions 0 .. L - Sq + t (bottom-right causal);
* a query that sees no position gets O = 0 and lse = -inf;
* logical token n of request b lives in row n % P of pool page
  ``page_table[b, n // P]``.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .e4m3 import decode_e4m3

D_KV = 576
D_V = 512


def gather_kv_rows(kv_pool8: np.ndarray, page_table: np.ndarray, b: int, n_tokens: int,
                   page_size: int) -> np.ndarray:
    """Bytes of request ``b``'s first ``n_tokens`` KV rows in logical order."""
    n = np.arange(n_tokens, dtype=np.int64)
    pages = page_table[b, n // page_size].astype(np.int64)
    flat = kv_pool8.reshape(-1, D_KV)
    return flat[pages * page_size + n % page_size]


def _softmax_rows(z: np.ndarray, vd: np.ndarray):
    """O = softmax(z) @ vd and lse = logsumexp(z), rows of z independent."""
    if z.shape[-1] == 0:
        return (np.zeros(z.shape[:-1] + (vd.shape[-1],)),
                np.full(z.shape[:-1], -np.inf))
    m = z.max(axis=-1, keepdims=True)
    w = np.exp(z - m)
    l = w.sum(axis=-1, keepdims=True)
    o = (w @ vd) / l
    return o, (m + np.log(l))[..., 0]


def attention_fp64(q8: np.ndarray, q_scale: float, kv_pool8: np.ndarray, kv_scale: float,
                   page_table: np.ndarray, seq_lens: np.ndarray, page_size: int,
                   softmax_scale: float, requests: Optional[Sequence[int]] = None,
                   heads: Optional[Sequence[int]] = None,
                   token_range: Optional[Sequence[int]] = None,
                   q_lens: Optional[Sequence[int]] = None):
    """Unsplit decode attention.

    q8: uint8 ``[B, Sq, H, 576]``; kv_pool8: uint8 ``[pages, P, 576]``;
    page_table: int32 ``[B, max_pages]``; seq_lens: ``[B]``.
    ``requests`` / ``heads`` restrict the work to a subset (the result keeps
    only those, in the given order).  ``token_range=(lo, hi)`` restricts every
    query to logical positions ``[lo, hi)`` intersected with its causal window
    (used to state one split of the split form).
    ``q_lens[b]`` (clamped to [0, Sq]) gives request b its own number of query tokens:
    they are the first q_lens[b] slots of ``q8[b]`` and the last q_lens[b] positions of
    its context (a verify step with a different number of draft tokens per request,
    [A/MLA] opening paragraph); the remaining slots see nothing (O = 0, lse = -inf).
    Returns ``(O [b, Sq, h, 512], lse [b, Sq, h])`` in float64.
    """
    B, Sq, H, _ = q8.shape
    reqs = list(range(B)) if requests is None else list(requests)
    hs = list(range(H)) if heads is None else list(heads)
    out = np.zeros((len(reqs), Sq, len(hs), D_V))
    lse = np.full((len(reqs), Sq, len(hs)), -np.inf)
    for i, b in enumerate(reqs):
        L = int(seq_lens[b])
        kd = decode_e4m3(gather_kv_rows(kv_pool8, page_table, b, L, page_size)) * float(kv_scale)
        vd = kd[:, :D_V]
        qd = decode_e4m3(q8[b][:, hs, :]) * float(q_scale)           # [Sq, h, 576]
        nq = Sq if q_lens is None else min(max(int(q_lens[b]), 0), Sq)
        for t in range(nq):
            hi = L - nq + t + 1                                        # visible: [0, hi)
            lo = 0
            if token_range is not None:
                lo, hi = max(lo, token_range[0]), min(hi, token_range[1])
            if hi <= lo:
                continue
            z = float(softmax_scale) * (qd[t] @ kd[lo:hi].T)            # [h, n]
            out[i, t], lse[i, t] = _softmax_rows(z, vd[lo:hi])
    return out, lse


def even_partition(seq_len: int, num_splits: int, align: int = 64):
    """Boundaries of ``num_splits`` contiguous chunks, each a multiple of ``align``
    tokens except the last; trailing chunks may be empty."""
    tiles = -(-seq_len // align)
    per = -(-tiles // num_splits) * align
    return [(min(s * per, seq_len), min((s + 1) * per, seq_len)) for s in range(num_splits)]


def split_partials_fp64(q8, q_scale, kv_pool8, kv_scale, page_table, seq_lens, page_size,
                        softmax_scale, bounds_per_request):
    """Per-chunk partial results: the unsplit definition restricted to each chunk.

    ``bounds_per_request[b]`` is a list of S ``(lo, hi)`` token ranges.
    Returns ``(O_s [B, S, Sq, H, 512], lse_s [B, S, Sq, H])``; an empty chunk
    has O_s = 0 and lse_s = -inf.
    """
    B, Sq, H, _ = q8.shape
    S = len(bounds_per_request[0])
    po = np.zeros((B, S, Sq, H, D_V))
    pl = np.full((B, S, Sq, H), -np.inf)
    for b in range(B):
        for s, rng in enumerate(bounds_per_request[b]):
            o, l = attention_fp64(q8, q_scale, kv_pool8, kv_scale, page_table, seq_lens,
                                  page_size, softmax_scale, requests=[b], token_range=rng)
            po[b, s], pl[b, s] = o[0], l[0]
    return po, pl


def combine_fp64(partial_o: np.ndarray, partial_lse: np.ndarray):
    """Log-sum-exp merge of split partials along axis 1 ([A/MLA] item (2)).

    M = max_s lse_s; w_s = exp(lse_s - M); O = sum_s w_s O_s / sum_s w_s;
    lse = M + log(sum_s w_s).  Rows whose partials are all empty give O = 0,
    lse = -inf.
    """
    m = partial_lse.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(partial_lse - m_safe[:, None])                    # exp(-inf) = 0
    den = w.sum(axis=1)
    num = (w[..., None] * partial_o).sum(axis=1)
    o = np.where(empty[..., None], 0.0, num / np.where(empty, 1.0, den)[..., None])
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, den)))
    return o, lse
