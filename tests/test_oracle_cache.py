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
