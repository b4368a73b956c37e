"""The parity checker itself (tests/oracle_side.check_output), on the CPU: what it lets through
and what it must reject.  Values are placed by hand so that each bound is met or missed by a
known margin."""
import numpy as np
import pytest

from tests import oracle_side as ors


def _bf16_rne(x):
    """bf16 round-to-nearest-even of float64 values, through their float32 bit patterns."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _ref(seed=0):
    rng = np.random.default_rng(seed)
    r = rng.normal(0.0, 0.3, size=(4, 512))
    r[0, :8] = [-4.01829597286237, 4.0183, 3.999, 2.7, 7.9, -6.3, 0.0, 1e-8]
    return r


def test_correctly_rounded_bf16_output_passes_at_every_magnitude():
    ref = _ref()
    out = _bf16_rne(ref)
    assert np.abs(out[0, 0] - ref[0, 0]) > 1e-2  # rounding alone exceeds the flat 1e-2 there
    ors.check_output(out, ref)


@pytest.mark.parametrize("x, half_ulp", [(0.5, 2.0 ** -9), (0.3, 2.0 ** -10), (1.5, 2.0 ** -8),
                                         (3.0, 2.0 ** -7), (5.0, 2.0 ** -6)])
def test_error_just_past_the_bound_fails_and_just_inside_passes(x, half_ulp):
    ref = np.zeros((2, 512))
    ref[0, 0] = x
    bound = 1e-2 + half_ulp
    ok = ref.copy()
    ok[0, 0] = x - 0.999 * bound  # toward zero: the ulp is taken at |ref|, the larger one
    ors.check_output(ok, ref, mean_rel=1.0)
    bad = ref.copy()
    bad[0, 0] = x - 1.001 * bound
    with pytest.raises(AssertionError, match="abs error"):
        ors.check_output(bad, ref, mean_rel=1.0)


def test_normalised_l1_bound_still_applies():
    ref = _ref(1)
    out = ref * (1.0 + 3e-3)  # every element 0.3 % off: max abs small, nL1 3e-3 > 2e-3
    with pytest.raises(AssertionError, match="normalised L1"):
        ors.check_output(out, ref)
    ors.check_output(ref * (1.0 + 1.5e-3), ref)


def test_non_finite_output_and_lse_mismatch_fail():
    ref = _ref(2)
    bad = ref.copy()
    bad[1, 3] = np.nan
    with pytest.raises(AssertionError, match="non-finite"):
        ors.check_output(bad, ref)
    lse_ref = np.array([1.0, -np.inf, 5.0])
    ors.check_output(ref, ref, np.array([1.0005, -np.inf, 5.0]), lse_ref)
    with pytest.raises(AssertionError):
        ors.check_output(ref, ref, np.array([1.0, 0.0, 5.0]), lse_ref)       # -inf expected
    with pytest.raises(AssertionError, match="lse error"):
        ors.check_output(ref, ref, np.array([1.0, -np.inf, 5.002]), lse_ref)  # 2e-3 > 1.15e-3
