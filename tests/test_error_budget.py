"""Error budget of the P.V precision (CPU only): why the decode computes P.V as two FP8 terms.

The oracle never rounds the softmax probabilities P; the decode multiplies them with the FP8
values V on FP8 matrix instructions, so P has to be encoded in 8-bit floats, and that
rounding counts against the accuracy contract (bf16 output: max abs error <= 1e-2,
sum|err| / sum|ref| <= 2e-3 against the fp64 oracle).  This study emulates, in float64 on the
host, the decode's arithmetic around P, with the oracle's own E4M3 encoder:

* scores in log2 units from the dequantised FP8 Q and KV;
* per query row a fixed reference mu = the largest score of the first 64-token step;
  per step a power-of-two exponent e = floor(step max - mu), and p = 2^(x - mu - e) * 224
  in fp32, so every p lies in [0, 448);
* P encoded one of four ways: exact (fp32), one e4m3 value (round to nearest even), one e4m3
  value with stochastic rounding (unbiased), or hi + lo with hi = e4m3(p) and
  lo = e4m3(p - hi) (two matrix instructions sharing V);
* O = sum_steps 2^e sum_i P_i V_i / sum_steps 2^e sum_i p_i (the sum of probabilities uses
  the exact p, as the kernel's fp32 running sum does), times the KV scale, rounded to bf16.

Inputs are the workloads' recipe: seeded N(0, 1) fp32 Q and KV, per-tensor scales, softmax
scale 1/sqrt(192), at 256, 4096 and 131072 positions.  The result that fixes the design: one
e4m3 P misses the 2e-3 bound at every length (stochastic rounding misses it by more), and
hi + lo meets it.
"""
import math

import numpy as np
import pytest

from oracle import attention_fp64, decode_e4m3, e4m3_table, per_tensor_scale, quantize_e4m3_sat
from synthetic import Workload, kv_request_f32, q_f32

SM = 1.0 / math.sqrt(192.0)
LOG2_224 = math.log2(224.0)
STEP = 64

_POS = e4m3_table()[:0x7F]  # non-negative finite e4m3 values, increasing


def _e4m3(x32: np.ndarray) -> np.ndarray:
    """Nearest-even e4m3 value of non-negative fp32 values below 464 (the oracle's encoder)."""
    return decode_e4m3(quantize_e4m3_sat(x32, np.float32(1.0)))


def _e4m3_stochastic(x32: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    """Unbiased stochastic rounding onto the non-negative e4m3 grid: the upper neighbour with
    probability (x - lower) / (upper - lower)."""
    a = x32.astype(np.float64)
    hi = np.minimum(np.searchsorted(_POS, a, side="left"), len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    lo = np.where(_POS[hi] == a, hi, lo)
    span = _POS[hi] - _POS[lo]
    frac = np.where(span > 0, (a - _POS[lo]) / np.where(span > 0, span, 1.0), 0.0)
    return np.where(rng.random(a.shape) < frac, _POS[hi], _POS[lo])


def _bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) -> float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def emulate(heads: int, L: int, seed: int):
    """Oracle output and the emulated decode output under each P encoding: a dict of
    (max abs error, normalised L1 error) against the oracle."""
    w = Workload("budget", batch=1, heads=heads, q_tokens=1, context=L, seed=seed)
    q = q_f32(w)
    kv = kv_request_f32(w, 0, L)
    qs, ks = per_tensor_scale(q), per_tensor_scale(kv)
    q8 = quantize_e4m3_sat(q, qs)
    kv8 = quantize_e4m3_sat(kv, ks, threads=8)
    del kv
    pool = np.zeros((1, L, 576), np.uint8)
    pool[0] = kv8
    o_ref, _ = attention_fp64(q8, qs, pool, ks, np.zeros((1, 1), np.int32),
                              np.array([L], np.int32), L, SM)
    o_ref = o_ref[0, 0]                                            # [H, 512]

    qd = decode_e4m3(q8[0, 0])                                     # [H, 576], code values
    kd = decode_e4m3(kv8)                                          # [L, 576]
    c2 = float(qs) * float(ks) * SM / math.log(2.0)
    z = c2 * (qd @ kd.T)                                           # [H, L], log2 units
    n_steps = L // STEP
    z = z.reshape(heads, n_steps, STEP)
    v = kd[:, :512].reshape(n_steps, STEP, 512)
    mu = z[:, 0].max(axis=1)                                       # first step's max
    e = np.clip(np.floor(z.max(axis=2) - mu[:, None]), -126, 127)  # [H, steps]
    p = np.exp2(z - (mu[:, None] + e)[:, :, None] + LOG2_224).astype(np.float32)
    scale = np.exp2(e)                                             # [H, steps]
    den = np.einsum("hs,hs->h", scale, p.astype(np.float64).sum(axis=2))

    rng = np.random.default_rng(seed + 1)
    hi = _e4m3(p)
    lo = _e4m3((p - hi.astype(np.float32)).astype(np.float32))
    encodings = {
        "fp32": p.astype(np.float64),
        "e4m3": hi,
        "e4m3_stochastic": _e4m3_stochastic(p, rng),
        "e4m3_hi_lo": hi + lo,
    }
    out = {}
    for name, pe in encodings.items():
        num = np.einsum("hs,hsk,skd->hd", scale, pe, v, optimize=True)
        o = _bf16((num / den[:, None]) * float(ks))
        err = np.abs(o - o_ref)
        out[name] = (float(err.max()), float(err.sum() / np.abs(o_ref).sum()))
    return out


CASES = [(16, 256, 0), (16, 4096, 0), (8, 131072, 0)]


@pytest.fixture(scope="module", params=CASES, ids=[f"L{c[1]}" for c in CASES])
def budget(request):
    heads, L, seed = request.param
    res = emulate(heads, L, seed)
    print(f"\nP.V error budget, L = {L}, {heads} heads (max abs / normalised L1): " +
          "; ".join(f"{k} {a:.2e} / {b:.2e}" for k, (a, b) in res.items()))
    return res


def test_hi_lo_meets_the_contract(budget):
    mx, nl1 = budget["e4m3_hi_lo"]
    assert mx <= 1e-2 and nl1 <= 2e-3


def test_fp32_p_meets_the_contract(budget):
    # the rest of the arithmetic (fp32 probabilities, bf16 output) leaves room for P's error
    mx, nl1 = budget["fp32"]
    assert mx <= 1e-2 and nl1 <= 2e-3


def test_single_e4m3_misses_the_bound(budget):
    assert budget["e4m3"][1] > 2e-3


def test_stochastic_rounding_misses_it_too(budget):
    # unbiased, but its spread is what the error consists of
    assert budget["e4m3_stochastic"][1] > budget["e4m3"][1] > 2e-3
