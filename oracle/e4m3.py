"""E4M3 decode and saturating quantisation, written from the definitions.

[A/MLA] item (4): the prep step converts Q and KV to FP8, and with saturation a
value outside the range is clamped to +-448 instead of turning into NaN.
[OCP]: E4M3 is sign-magnitude with 4 exponent bits (bias 7) and 3 mantissa
bits; exponent field 0 holds subnormals; S.1111.111 is NaN; there is no
infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.

Readings taken where neither source is explicit:

* rounding is to the nearest representable value, ties to the even code
  (IEEE's default);
* the value quantised is the fp32 quotient ``float32(x) / float32(scale)``
  (IEEE division), so a per-tensor scale s = amax / 448 maps amax to 448;
* NaN stays NaN and keeps its sign: code ``0x7F | sign``;
* +-inf and every finite |t| >= 448 saturate to ``0x7E | sign``;
* the sign of zero is kept (-0 and negatives that round to 0 give 0x80).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_table() -> np.ndarray:
    """Value of every one of the 256 codes, float64 (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * 2.0 ** -6 * (man / 8.0)
        else:
            vals[code] = sign * 2.0 ** (exp - 7) * (1.0 + man / 8.0)
    return vals


_TABLE = e4m3_table()
# Non-negative finite values in code order 0x00 .. 0x7E; strictly increasing.
_POS = _TABLE[:0x7F].copy()


def decode_e4m3(codes) -> np.ndarray:
    """Bytes -> float64 through the table."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def per_tensor_scale(x) -> np.float32:
    """Per-tensor dequantisation scale float32(max|x|) / float32(448); 1 if max|x| = 0."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32))))
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def _quantize_chunk(t: np.ndarray) -> np.ndarray:
    """Codes of fp32 quotients t: clamp |t| to 448 (saturation), then the nearest value of the
    non-negative grid, ties to the even code; NaN -> 0x7F; the sign bit is copied."""
    a = np.minimum(np.abs(t), np.float32(E4M3_MAX)).astype(np.float64)  # NaN stays NaN
    hi = np.searchsorted(_POS, a, side="left")          # _POS[hi-1] < a <= _POS[hi]
    np.minimum(hi, len(_POS) - 1, out=hi)               # only NaN lands past the end
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))   # exact hit: d_hi == 0
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code[np.isnan(t)] = 0x7F
    return code | (np.signbit(t).astype(np.uint8) << 7)


def quantize_e4m3_sat(x, scale, threads: int = 0) -> np.ndarray:
    """Saturating round-to-nearest-even encode of ``float32(x) / float32(scale)``.

    The nearest value is found by searching the table of non-negative finite codes;
    distances are exact in float64 because both neighbours lie within a factor of two of
    the input (or the lower one is 0).  Large inputs are processed in independent chunks,
    on ``threads`` worker threads if given (elementwise, so the result does not depend on
    the chunking).
    """
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        t = np.asarray(np.asarray(x, dtype=np.float32) / np.float32(scale), dtype=np.float32)
    flat = t.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 22
    spans = [(i, min(i + step, flat.size)) for i in range(0, flat.size, step)]

    def run(span):
        out[span[0]:span[1]] = _quantize_chunk(flat[span[0]:span[1]])

    if threads and threads > 1 and len(spans) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, spans))
    else:
        for sp in spans:
            run(sp)
    return out.reshape(t.shape)
