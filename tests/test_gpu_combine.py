"""GPU LSE combine in isolation on oracle-made partials (runs on an MI355X).

The combine's inputs are fp16 partial rows in units of the KV scale (what the decode kernel
writes), so the partials are rounded to fp16 here first and the oracle merges exactly those
values; the GPU result may differ from it only by fp32 accumulation and the bf16 rounding of
the output.
"""
import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from oracle import combine_fp64
from tests.oracle_side import bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,S,Sq,H", [(1, 1, 1, 16), (2, 3, 2, 16), (1, 64, 1, 128),
                                      (3, 100, 1, 32), (1, 17, 8, 16), (1, 256, 1, 128)])
def test_combine_matches_oracle(B, S, Sq, H):
    rng = np.random.default_rng(S * 7 + H)
    R = Sq * H
    v_scale = np.float32(0.0123)
    po = (rng.standard_normal((B, S, R, 512)) * 60).astype(np.float16)   # |x| well inside 448
    pl = (rng.standard_normal((B, S, R)) * 4).astype(np.float32)
    if S > 1:
        pl[:, ::3, :] = -np.inf                      # empty splits ...
        po[:, ::3, :, :] = np.nan                    # ... whose partial values are garbage
    pl[0, :, 0] = -np.inf                            # a row with nothing visible
    po64 = np.where(np.isnan(po), 0, po).astype(np.float64) * float(v_scale)
    o_ref, l_ref = combine_fp64(po64, pl.astype(np.float64))
    out, lse = mla.splitkv_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                                   Sq, H, float(v_scale))
    o = bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(B, R, 512)
    o_ref = o_ref.reshape(B, R, 512)
    # bf16 rounding of the exact merge plus fp32 accumulation
    assert np.all(np.abs(o - o_ref) <= np.abs(o_ref) * 2.0 ** -8 + 1e-6)
    assert np.all(o[0, 0] == 0)
    lse = lse.cpu().numpy().reshape(B, R)
    fin = np.isfinite(l_ref.reshape(B, R))
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - l_ref.reshape(B, R)[fin])) <= 1e-5


@pytest.mark.parametrize("S,H", [(1024, 32), (4096, 32)])
def test_combine_many_splits_both_outputs(S, H):
    """Up to the largest split count the combine accepts, with empty splits among them: the
    bf16 output and the merged partial (fp16 in units of v_scale) against the oracle's merge
    of the same values."""
    rng = np.random.default_rng(S + H)
    B, R = 1, H
    v_scale = np.float32(0.02)
    po = (rng.standard_normal((B, S, R, 512)) * 60).astype(np.float16)
    pl = (rng.standard_normal((B, S, R)) * 6).astype(np.float32)
    pl[:, 5::7, :] = -np.inf
    po[:, 5::7, :, :] = np.nan
    po64 = np.where(np.isnan(po), 0, po).astype(np.float64)
    o_ref, l_ref = combine_fp64(po64, pl.astype(np.float64))          # units of v_scale
    gpo, gpl = torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda()
    out, lse = mla.splitkv_combine(gpo, gpl, 1, H, float(v_scale))
    mo = torch.empty((B, R, 512), dtype=torch.float16, device="cuda")
    ml = torch.empty((B, R), dtype=torch.float32, device="cuda")
    mla.splitkv_combine_partial(gpo, gpl, 1, H, mo, ml)
    torch.cuda.synchronize()
    o = bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(B, R, 512)
    ref = o_ref.reshape(B, R, 512) * float(v_scale)
    assert np.all(np.abs(o - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)
    m = mo.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(m - o_ref.reshape(B, R, 512)) <= np.abs(o_ref.reshape(B, R, 512))
                  * 2.0 ** -10 + 1e-4)
    for got in (lse.cpu().numpy().reshape(B, R), ml.cpu().numpy()):
        assert np.max(np.abs(got - l_ref.reshape(B, R))) <= 1e-4


def _sweep_cases(seed=20261207):
    """Split counts on every side of the kernel's batch and wave-count choices (8, 16, 32,
    64 and 512 splits per row, up to 16 waves), with random batch, query tokens and heads."""
    rng = np.random.default_rng(seed)
    counts = [2, 4, 8, 9, 12, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 127, 128, 129,
              255, 257, 511, 512, 513, 700, 1000, 2048, 4095]
    out = []
    for i, S in enumerate(counts):
        H = int(rng.choice([1, 8, 16, 24, 128] if S <= 512 else [1, 8, 16]))
        Sq = int(rng.integers(1, 5)) if H <= 24 else 1
        B = int(rng.integers(1, 4)) if S <= 512 else 1
        out.append((f"s{S}_b{B}_sq{Sq}_h{H}", B, S, Sq, H, int(rng.integers(0, 1 << 30))))
    return out


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[c[0] for c in SWEEP])
def test_combine_sweep_both_outputs(case):
    """Random empty splits (their values NaN) and rows with no live split, against the
    oracle's merge of the same fp16 values: the bf16 output, and the merged partial written
    as slice 1 of a [B, 2, R] buffer (slice 0 untouched)."""
    name, B, S, Sq, H, seed = case
    print(f"[combine] {name}", flush=True)
    rng = np.random.default_rng(seed)
    R = Sq * H
    v_scale = np.float32(rng.uniform(1e-3, 0.05))
    po = (rng.standard_normal((B, S, R, 512)) * 60).astype(np.float16)
    pl = (rng.standard_normal((B, S, R)) * rng.uniform(0.5, 20)).astype(np.float32)
    empty = rng.random((B, S, R)) < 0.3
    pl[empty] = -np.inf
    po[empty] = np.nan
    pl[:, :, int(rng.integers(0, R))] = -np.inf       # one row that sees nothing
    po64 = np.where(np.isnan(po), 0, po).astype(np.float64)
    o_ref, l_ref = combine_fp64(po64, pl.astype(np.float64))           # units of v_scale
    gpo, gpl = torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda()
    out, lse = mla.splitkv_combine(gpo, gpl, Sq, H, float(v_scale))
    mo = torch.full((B, 2, R, 512), float("nan"), dtype=torch.float16, device="cuda")
    ml = torch.full((B, 2, R), float("nan"), dtype=torch.float32, device="cuda")
    mla.splitkv_combine_partial(gpo, gpl, Sq, H, mo[:, 1], ml[:, 1], 2 * R)
    torch.cuda.synchronize()
    o = bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(B, R, 512)
    ref = o_ref.reshape(B, R, 512) * float(v_scale)
    assert np.all(np.abs(o - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)
    m = mo[:, 1].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(m - o_ref.reshape(B, R, 512)) <= np.abs(o_ref.reshape(B, R, 512))
                  * 2.0 ** -10 + 1e-4)
    assert torch.isnan(mo[:, 0].float()).all() and torch.isnan(ml[:, 0]).all()
    fin = np.isfinite(l_ref.reshape(B, R))
    for got in (lse.cpu().numpy().reshape(B, R), ml[:, 1].cpu().numpy()):
        assert np.array_equal(fin, np.isfinite(got))
        if fin.any():  # (a single row that sees nothing leaves no finite lse)
            assert np.max(np.abs(got[fin] - l_ref.reshape(B, R)[fin])) <= 1e-4
