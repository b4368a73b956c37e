"""Pins for the oracle's E4M3 table and saturating quantiser (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import decode_e4m3, e4m3_table, per_tensor_scale, quantize_e4m3_sat
from tests.conftest import read_golden


def _lib_cast_saturating(t32: np.ndarray) -> np.ndarray:
    """torch's RNE float8_e4m3fn cast after a clamp to +-448 (the library route)."""
    t = torch.from_numpy(np.ascontiguousarray(t32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _structured_fp32(n_random=1 << 20, seed=7):
    """Every 16-bit high half with four low halves (0, tie bit, just below, all ones)
    plus uniformly random bit patterns: covers every exponent and every rounding case."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x8000, 0x7FFF, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(seed).integers(0, 1 << 32, size=n_random, dtype=np.uint64)
    return np.concatenate([pats, rnd.astype(np.uint32)]).view(np.float32)


def test_table_spot_values_from_spec():
    tab = e4m3_table()
    for code, val, *_ in read_golden("e4m3_points.txt"):
        c = int(code, 16)
        if val == "nan":
            assert np.isnan(tab[c])
        else:
            assert tab[c] == float(val), (code, tab[c], val)
            assert np.signbit(tab[c]) == val.startswith("-")


def test_table_equals_torch_float8_e4m3fn():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    tab = e4m3_table()
    same = (tab == lib) | (np.isnan(tab) & np.isnan(lib))
    assert same.all(), np.nonzero(~same)


def test_table_is_monotonic_on_positive_codes():
    pos = e4m3_table()[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0


def test_quantize_hand_worked_ties_and_saturation():
    for x, code, *_ in read_golden("e4m3_rounding.txt"):
        got = quantize_e4m3_sat(np.array([float(x)], dtype=np.float32), 1.0)[0]
        assert got == int(code, 16), (x, hex(got), code)


def test_quantize_equals_library_on_structured_sweep():
    x = _structured_fp32()
    got = quantize_e4m3_sat(x, 1.0)
    nan = np.isnan(x)
    ref = _lib_cast_saturating(np.where(nan, 0, x).astype(np.float32))
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN keeps its sign: 0x7F | sign
    assert np.array_equal(got[nan], np.where(np.signbit(x[nan]), 0xFF, 0x7F).astype(np.uint8))


def test_saturation_never_produces_nan():
    x = np.array([448.0, 449.0, 464.0, 465.0, 480.0, 1e4, 3.4e38, np.inf,
                  -449.0, -1e30, -np.inf], dtype=np.float32)
    q = quantize_e4m3_sat(x, 1.0)
    assert np.all((q & 0x7F) == 0x7E)
    assert np.array_equal(q >> 7, np.signbit(x).astype(np.uint8))


def test_quantize_divides_by_scale_in_fp32():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200_000).astype(np.float32)
    s = per_tensor_scale(x)
    q = quantize_e4m3_sat(x, s)
    # the scale maps amax exactly onto the top code
    i = np.argmax(np.abs(x))
    assert (q[i] & 0x7F) == 0x7E
    # quantising x with scale s equals quantising the fp32 quotient with scale 1
    assert np.array_equal(q, quantize_e4m3_sat(x / np.float32(s), 1.0))
    # and the decoded value is within half a step of the quotient
    t = (x / np.float32(s)).astype(np.float64)
    d = decode_e4m3(q)
    assert np.all(np.abs(d - t) <= np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_per_tensor_scale():
    assert per_tensor_scale(np.zeros(8, np.float32)) == np.float32(1.0)
    x = np.array([1.0, -896.0, 3.0], dtype=np.float32)
    assert per_tensor_scale(x) == np.float32(2.0)
    assert per_tensor_scale(x).dtype == np.float32


def test_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(quantize_e4m3_sat(vals, 1.0), codes)


@pytest.mark.slow
def test_quantize_exhaustive_all_fp32_patterns():
    """All 2^32 fp32 bit patterns against the library route (opt-in, minutes)."""
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        x = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32).view(np.float32)
        nan = np.isnan(x)
        got = quantize_e4m3_sat(x, 1.0)
        ref = _lib_cast_saturating(np.where(nan, 0, x).astype(np.float32))
        assert np.array_equal(got[~nan], ref[~nan]), hex(start)
