"""Pins for the oracle's cache preparation: bf16 decoding, data-derived scales and the
paged KV append (CPU only)."""
import numpy as np
import torch

from oracle import (append_kv_fp8, bf16_bits_to_f32, dynamic_quantize, gather_kv_rows,
                    per_tensor_scale, quantize_e4m3_sat)


def test_bf16_bits_equal_torch_conversion_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = bf16_bits_to_f32(bits)
    same = (got.view(np.uint32) == lib.view(np.uint32)) | (np.isnan(got) & np.isnan(lib))
    assert same.all()


def test_bf16_spot_values():
    got = bf16_bits_to_f32(np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x8000], np.uint16))
    assert got[0] == 1.0 and got[1] == -2.0 and np.isinf(got[2]) and got[2] > 0
    assert got[3] == np.float32(2.0 ** -133)          # smallest bf16 subnormal
    assert got[4] == 0 and np.signbit(got[4])


def test_dynamic_scale_maps_amax_to_the_largest_code():
    rng = np.random.default_rng(3)
    for scale_up in (1e-30, 1e-3, 1.0, 7.5, 1e30):
        x = (rng.standard_normal(4097) * scale_up).astype(np.float32)
        codes, s = dynamic_quantize(x)
        i = int(np.argmax(np.abs(x)))
        assert codes[i] & 0x7F == 0x7E
        assert s == np.float32(np.abs(x).max()) / np.float32(448)
        # nothing saturates beyond the largest code and nothing turns into NaN
        assert not np.any((codes & 0x7F) == 0x7F)


def test_dynamic_scale_of_zeros_is_one():
    codes, s = dynamic_quantize(np.zeros(100, np.float32))
    assert s == 1.0 and not codes.any()


def test_bf16_source_agrees_with_the_same_values_in_fp32():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(10000).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)        # truncation to bf16
    c16, s16 = dynamic_quantize(bits, source="bf16")
    x_trunc = (bits.astype(np.uint32) << 16).view(np.float32)
    c32, s32 = dynamic_quantize(x_trunc)
    assert s16 == s32 and np.array_equal(c16, c32)
    # and with a hand scale: the encode of the decoded values
    assert np.array_equal(c16, quantize_e4m3_sat(x_trunc, per_tensor_scale(x_trunc)))


def _pool_case(rng, batch=3, page_size=8, lens=(1, 13, 40)):
    """A permuted page pool with room for every request's full length."""
    max_pages = max((L + page_size - 1) // page_size for L in lens) + 1
    num_pages = batch * max_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    page_table = perm.reshape(batch, max_pages)
    pool = rng.integers(0, 256, size=(num_pages, page_size, 576), dtype=np.uint8)
    return pool, page_table, max_pages


def test_step_by_step_append_reads_back_through_the_attention_gather():
    rng = np.random.default_rng(5)
    lens = (1, 13, 40)
    pool, page_table, _ = _pool_case(rng, lens=lens)
    s = np.float32(0.01)
    kv = [rng.standard_normal((L, 576)).astype(np.float32) for L in lens]
    for step in range(max(lens)):
        # every request that still has tokens appends one; a finished request is given a
        # length past its page table, so its (repeated) last row must not be written
        seq = np.array([min(step + 1, L) for L in lens], np.int32)
        new = np.stack([kv[b][min(step, L - 1)] for b, L in enumerate(lens)])[:, None]
        for b, L in enumerate(lens):
            if step >= L:
                seq[b] = 10 ** 6                               # past the table: skipped
        pool = append_kv_fp8(pool, page_table, seq, new, s)
    for b, L in enumerate(lens):
        got = gather_kv_rows(pool, page_table, b, L, 8)
        assert np.array_equal(got, quantize_e4m3_sat(kv[b], s)), b


def test_append_touches_only_the_new_rows():
    rng = np.random.default_rng(6)
    pool, page_table, max_pages = _pool_case(rng)
    seq = np.array([5, 17, 24], np.int32)
    new = rng.standard_normal((3, 4, 576)).astype(np.float32)
    out = append_kv_fp8(pool, page_table, seq, new, np.float32(0.02))
    changed = np.zeros(pool.shape[:2], bool)
    for b in range(3):
        for t in range(4):
            n = seq[b] - 4 + t
            changed[page_table[b, n // 8], n % 8] = True
    assert np.array_equal(out[~changed], pool[~changed])
    assert changed.sum() == 12


def test_t_row_append_equals_t_single_appends():
    rng = np.random.default_rng(7)
    pool, page_table, _ = _pool_case(rng)
    seq = np.array([4, 20, 33], np.int32)
    new = rng.standard_normal((3, 4, 576)).astype(np.float32)
    s = np.float32(0.005)
    once = append_kv_fp8(pool, page_table, seq, new, s)
    step = pool
    for t in range(4):
        step = append_kv_fp8(step, page_table, seq - 3 + t, new[:, t:t + 1], s)
    assert np.array_equal(once, step)


def test_out_of_range_positions_and_pages_are_skipped():
    rng = np.random.default_rng(8)
    pool, page_table, max_pages = _pool_case(rng)
    pt = page_table.copy()
    pt[1, :] = -1                                              # request 1: no valid page
    seq = np.array([1, 9, max_pages * 8 + 2], np.int32)        # request 2: past the table
    new = rng.standard_normal((3, 2, 576)).astype(np.float32)
    out = append_kv_fp8(pool, pt, seq, new, np.float32(0.1))
    # request 0: position -1 skipped, position 0 written
    assert np.array_equal(out[pt[0, 0], 0], quantize_e4m3_sat(new[0, 1], np.float32(0.1)))
    mask = np.ones(pool.shape[:2], bool)
    mask[pt[0, 0], 0] = False
    assert np.array_equal(out[mask], pool[mask])


# ---- RoPE fused with the append ---------------------------------------------------------

from oracle import append_kv_rope_fp8, rope_rotate_f32  # noqa: E402


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(np.maximum(x, np.float32(np.finfo(np.float32).tiny)))


def test_rope_rotation_is_the_complex_product_within_three_roundings():
    """Against the rotation of the same fp32 inputs in fp64 (products exact there): each
    rotated value is within half an ulp of each of its two products and of itself."""
    rng = np.random.default_rng(21)
    for _ in range(50):
        row = (rng.standard_normal(576) * rng.choice([1e-3, 1.0, 50.0])).astype(np.float32)
        ang = rng.uniform(-np.pi, np.pi, 32)
        c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
        got = rope_rotate_f32(row, c, s)
        x0, x1 = row[512::2].astype(np.float64), row[513::2].astype(np.float64)
        c64, s64 = c.astype(np.float64), s.astype(np.float64)
        ex0, ex1 = x0 * c64 - x1 * s64, x0 * s64 + x1 * c64
        b0 = 0.5 * (_ulp32(x0 * c64) + _ulp32(x1 * s64) + _ulp32(ex0)) * 1.0001
        b1 = 0.5 * (_ulp32(x0 * s64) + _ulp32(x1 * c64) + _ulp32(ex1)) * 1.0001
        assert np.all(np.abs(got[512::2] - ex0) <= b0)
        assert np.all(np.abs(got[513::2] - ex1) <= b1)
        assert np.array_equal(got[:512], row[:512])          # latent columns untouched


def test_rope_special_angles():
    rng = np.random.default_rng(22)
    row = rng.standard_normal(576).astype(np.float32)
    one, zero = np.ones(32, np.float32), np.zeros(32, np.float32)
    assert np.array_equal(rope_rotate_f32(row, one, zero), row)          # angle 0
    q = rope_rotate_f32(row, zero, one)                                 # a quarter turn
    assert np.array_equal(q[512::2], -row[513::2]) and np.array_equal(q[513::2], row[512::2])
    h = rope_rotate_f32(row, -one, zero)                                # half a turn
    assert np.array_equal(h[512:], -row[512:])


def test_rope_with_a_standard_table_matches_torch_complex_product():
    """A standard RoPE table (theta_i = 10000^(-2i/64), angle n theta_i) applied as the
    complex product of adjacent column pairs, as torch computes it in float64."""
    pos = np.arange(300)
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)
    ang = pos[:, None] * theta[None, :]
    cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    rng = np.random.default_rng(23)
    rows = rng.standard_normal((300, 576)).astype(np.float32)
    got = np.stack([rope_rotate_f32(rows[n], cos_t[n], sin_t[n]) for n in range(300)])
    z = torch.view_as_complex(torch.from_numpy(rows[:, 512:].astype(np.float64)).reshape(300, 32, 2))
    w = torch.complex(torch.from_numpy(cos_t.astype(np.float64)), torch.from_numpy(sin_t.astype(np.float64)))
    ref = torch.view_as_real(z * w).reshape(300, 64).numpy()
    assert np.max(np.abs(got[:, 512:] - ref)) <= 4 * np.finfo(np.float32).eps * np.abs(ref).max()


def test_rope_append_writes_the_rotated_rows_and_nothing_past_the_table():
    rng = np.random.default_rng(24)
    lens = np.array([2, 13, 40], np.int32)
    pool, page_table, _ = _pool_case(rng, lens=tuple(int(x) for x in lens))
    T = 3
    new = (rng.standard_normal((3, T, 576)) * 2).astype(np.float32)
    n_pos = int(lens.max()) - 1                  # the last position of the longest request is past it
    ang = rng.uniform(-np.pi, np.pi, (n_pos, 32))
    cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    scale = np.float32(0.01)
    got = append_kv_rope_fp8(pool, page_table, lens, new, scale, cos_t, sin_t)
    P = pool.shape[1]
    touched = np.zeros(pool.shape[:2], bool)
    for b in range(3):
        for t in range(T):
            n = int(lens[b]) - T + t
            if n < 0:
                continue
            page, r = page_table[b, n // P], n % P
            if n >= n_pos:
                assert np.array_equal(got[page, r], pool[page, r])     # past the table
                continue
            touched[page, r] = True
            want = quantize_e4m3_sat(rope_rotate_f32(new[b, t], cos_t[n], sin_t[n]), scale)
            assert np.array_equal(got[page, r], want)
            # the latent part is the plain append's
            plain = append_kv_fp8(pool, page_table, lens, new, scale)
            assert np.array_equal(got[page, r, :512], plain[page, r, :512])
    assert np.array_equal(got[~touched], pool[~touched])
