"""Pins for the oracle's attention, split partials and combine (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import (attention_fp64, combine_fp64, decode_e4m3, even_partition,
                    per_tensor_scale, quantize_e4m3_sat, split_partials_fp64)
from synthetic import WORKLOADS, kv_request_f32, page_layout, q_f32, seq_lens_for

SM = 1.0 / math.sqrt(192.0)


def _contig(kv8_rows_per_req):
    """Contiguous pool (one page per request) from a list of [L_b, 576] byte arrays."""
    P = max(-(-len(r) // 64) * 64 for r in kv8_rows_per_req)
    pool = np.full((len(kv8_rows_per_req), P, 576), 0x7F, dtype=np.uint8)  # NaN-poisoned tail
    for b, r in enumerate(kv8_rows_per_req):
        pool[b, :len(r)] = r
    table = np.arange(len(kv8_rows_per_req), dtype=np.int32)[:, None]
    return pool, table, P


def _rand_case(B=2, Sq=1, H=4, L=(70, 5), seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, 576)).astype(np.float32)
    kvs = [rng.standard_normal((Lb, 576)).astype(np.float32) for Lb in L]
    qs = per_tensor_scale(q)
    ks = per_tensor_scale(np.concatenate(kvs))
    q8 = quantize_e4m3_sat(q, qs)
    kv8 = [quantize_e4m3_sat(k, ks) for k in kvs]
    pool, table, P = _contig(kv8)
    return q8, qs, kv8, ks, pool, table, P, np.array(L, dtype=np.int32)


def _e4m3(v):
    """Byte of an exactly representable value (for hand-built inputs)."""
    return quantize_e4m3_sat(np.array([v], np.float32), 1.0)[0]


# ---------------------------------------------------------------- closed forms

def test_single_token_returns_its_value_row_and_score():
    q8, qs, kv8, ks, pool, table, P, _ = _rand_case(B=1, H=3, L=(1,))
    o, lse = attention_fp64(q8, qs, pool, ks, table, np.array([1], np.int32), P, SM)
    v0 = decode_e4m3(kv8[0][0]) * float(ks)
    assert np.array_equal(o[0, 0], np.broadcast_to(v0[:512], (3, 512)))
    z0 = SM * (decode_e4m3(q8[0, 0]) * float(qs)) @ v0          # v0 is the full 576 row here
    assert np.allclose(lse[0, 0], z0, rtol=0, atol=1e-12)


def test_two_keys_weights_are_logistic_in_the_score_gap():
    # q has one nonzero channel c; K rows differ only there -> z gap = SM*q_c*(k1_c-k0_c)
    c = 100
    q8 = np.zeros((1, 1, 1, 576), np.uint8)
    q8[0, 0, 0, c] = _e4m3(4.0)
    kv = np.zeros((2, 576), np.uint8)
    kv[0, c], kv[1, c] = _e4m3(1.0), _e4m3(3.0)
    kv[0, 7], kv[1, 7] = _e4m3(2.0), _e4m3(-0.5)                 # value column 7
    pool, table, P = _contig([kv])
    o, lse = attention_fp64(q8, 1.0, pool, 1.0, table, np.array([2], np.int32), P, SM)
    dz = SM * 4.0 * (3.0 - 1.0)
    w1 = 1.0 / (1.0 + math.exp(-dz))
    assert abs(o[0, 0, 0, 7] - ((1 - w1) * 2.0 + w1 * -0.5)) < 1e-14
    assert abs(o[0, 0, 0, c] - ((1 - w1) * 1.0 + w1 * 3.0)) < 1e-14
    z0, z1 = SM * 4.0 * 1.0, SM * 4.0 * 3.0
    assert abs(lse[0, 0, 0] - math.log(math.exp(z0) + math.exp(z1))) < 1e-14


def test_identical_rows_give_that_row():
    q8, qs, kv8, ks, _, _, _, _ = _rand_case(B=1, H=2, L=(1,))
    rows = np.repeat(kv8[0][:1], 37, axis=0)
    pool, table, P = _contig([rows])
    o, _ = attention_fp64(q8, qs, pool, ks, table, np.array([37], np.int32), P, SM)
    v0 = decode_e4m3(rows[0, :512]) * float(ks)
    assert np.allclose(o[0, 0], v0, rtol=0, atol=1e-14)


def test_dominant_key_wins_within_exp_of_the_lead():
    c = 5
    q8 = np.zeros((1, 1, 1, 576), np.uint8)
    q8[0, 0, 0, c] = _e4m3(448.0)
    kv = np.zeros((4, 576), np.uint8)
    kv[:, 300] = [_e4m3(v) for v in (1.0, 2.0, 3.0, 4.0)]
    kv[2, c] = _e4m3(0.875)                                      # lead of 448*0.875*SM ~ 28
    pool, table, P = _contig([kv])
    o, _ = attention_fp64(q8, 1.0, pool, 1.0, table, np.array([4], np.int32), P, SM)
    lead = 448.0 * 0.875 * SM
    assert abs(o[0, 0, 0, 300] - 3.0) < 4 * math.exp(-lead) * 4


def test_causal_window_is_bottom_right():
    q8, qs, kv8, ks, pool, table, P, _ = _rand_case(B=1, Sq=2, H=2, L=(2,))
    o, lse = attention_fp64(q8, qs, pool, ks, table, np.array([2], np.int32), P, SM)
    v = decode_e4m3(kv8[0]) * float(ks)
    # token 0 sees only position 0
    assert np.array_equal(o[0, 0], np.broadcast_to(v[0, :512], (2, 512)))
    # token 1 sees positions 0 and 1
    qd = decode_e4m3(q8[0, 1]) * float(qs)
    z = SM * qd @ v.T
    w = np.exp(z - z.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    assert np.allclose(o[0, 1], w @ v[:, :512], rtol=0, atol=1e-13)


# ------------------------------------------------------------- library check

def _sdpa_reference(q8, qs, kv8_list, ks, Sq):
    """float64 scaled_dot_product_attention with an explicit bottom-right mask;
    dequantisation through torch's float8_e4m3fn (independent of the oracle)."""
    outs, lses = [], []
    for b, rows in enumerate(kv8_list):
        L = rows.shape[0]
        k = torch.from_numpy(rows).view(torch.float8_e4m3fn).double() * float(ks)
        q = torch.from_numpy(np.ascontiguousarray(q8[b])).view(torch.float8_e4m3fn).double() * float(qs)
        q = q.permute(1, 0, 2)                                   # [H, Sq, 576]
        mask = torch.ones(Sq, L, dtype=torch.bool)
        for t in range(Sq):
            mask[t, L - Sq + t + 1:] = False
        kk = k[None].expand(q.shape[0], L, 576)
        vv = k[None, :, :512].expand(q.shape[0], L, 512)
        o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=SM)
        z = SM * q @ kk.transpose(1, 2)
        z = z.masked_fill(~mask, -math.inf)
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(torch.logsumexp(z, dim=-1).permute(1, 0).numpy())
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("Sq,L", [(1, (70, 5)), (3, (130, 4)), (8, (300, 8))])
def test_matches_torch_sdpa_float64(Sq, L):
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=len(L), Sq=Sq, H=4, L=L, seed=Sq)
    o, lse = attention_fp64(q8, qs, pool, ks, table, lens, P, SM)
    ro, rl = _sdpa_reference(q8, qs, kv8, ks, Sq)
    assert np.max(np.abs(o - ro)) <= 1e-12
    assert np.max(np.abs(lse - rl)) <= 1e-12


def test_matches_torch_sdpa_on_tiny_workload_and_4k_context():
    w = WORKLOADS["tiny"]
    lens = seq_lens_for(w)
    q = q_f32(w)
    kv = kv_request_f32(w, 0, int(lens[0]))
    qs, ks = per_tensor_scale(q), per_tensor_scale(kv)
    q8, kv8 = quantize_e4m3_sat(q, qs), quantize_e4m3_sat(kv, ks)
    pool, table, P = _contig([kv8])
    o, lse = attention_fp64(q8, qs, pool, ks, table, lens, P, SM)
    ro, rl = _sdpa_reference(q8, qs, [kv8], ks, 1)
    assert np.max(np.abs(o - ro)) <= 1e-12 and np.max(np.abs(lse - rl)) <= 1e-12
    q8b, qsb, kv8b, ksb, poolb, tableb, Pb, lensb = _rand_case(B=1, H=2, L=(4096,), seed=11)
    o, lse = attention_fp64(q8b, qsb, poolb, ksb, tableb, lensb, Pb, SM)
    ro, rl = _sdpa_reference(q8b, qsb, kv8b, ksb, 1)
    assert np.max(np.abs(o - ro)) <= 1e-12 and np.max(np.abs(lse - rl)) <= 1e-12


# ---------------------------------------------------------------- invariants

def test_paged_pool_equals_contiguous():
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=3, Sq=2, H=3, L=(200, 64, 129), seed=4)
    o_ref, l_ref = attention_fp64(q8, qs, pool, ks, table, lens, P, SM)
    page = 32
    n_pages = [-(-int(L) // page) for L in lens]
    perm = np.random.default_rng(9).permutation(sum(n_pages))
    ppool = np.full((sum(n_pages), page, 576), 0x7F, np.uint8)
    ptab = np.zeros((3, max(n_pages)), np.int32)
    off = 0
    for b, rows in enumerate(kv8):
        for j in range(n_pages[b]):
            pg = perm[off + j]
            ptab[b, j] = pg
            chunk = rows[j * page:(j + 1) * page]
            ppool[pg, :len(chunk)] = chunk
        off += n_pages[b]
    o, l = attention_fp64(q8, qs, ppool, ks, ptab, lens, page, SM)
    assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)


def test_heads_are_independent():
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=2, Sq=2, H=6, L=(90, 33), seed=5)
    o, l = attention_fp64(q8, qs, pool, ks, table, lens, P, SM)
    o2, l2 = attention_fp64(q8, qs, pool, ks, table, lens, P, SM, heads=[4, 1], requests=[1])
    assert np.array_equal(o2[0], o[1][:, [4, 1]]) and np.array_equal(l2[0], l[1][:, [4, 1]])


def test_workload_page_layout_is_a_permutation():
    w = WORKLOADS["paged_b32"]
    lens = seq_lens_for(w)
    assert lens.min() >= 4096 and lens.max() <= 131072
    P, table, n = page_layout(w, lens)
    used = np.concatenate([table[b, :-(-int(L) // P)] for b, L in enumerate(lens)])
    assert P == 64 and n == used.size and np.array_equal(np.sort(used), np.arange(n))


@pytest.mark.parametrize("S", [1, 2, 3, 4, 7, 64])
def test_split_count_does_not_change_the_result(S):
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=2, Sq=3, H=3, L=(700, 64), seed=6)
    o_ref, l_ref = attention_fp64(q8, qs, pool, ks, table, lens, P, SM)
    bounds = [even_partition(int(L), S, 64) for L in lens]
    po, pl = split_partials_fp64(q8, qs, pool, ks, table, lens, P, SM, bounds)
    o, l = combine_fp64(po, pl)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
    assert np.max(np.abs(l - l_ref)) <= 1e-12


def test_combine_single_split_is_identity():
    rng = np.random.default_rng(2)
    po = rng.standard_normal((2, 1, 3, 4, 512))
    pl = rng.standard_normal((2, 1, 3, 4))
    o, l = combine_fp64(po, pl)
    assert np.allclose(o, po[:, 0], rtol=0, atol=1e-15) and np.array_equal(l, pl[:, 0])


def test_combine_two_split_closed_form_and_empty_splits():
    rng = np.random.default_rng(8)
    o1, o2 = rng.standard_normal(512), rng.standard_normal(512)
    l1, l2 = 3.0, 1.5
    po = np.stack([o1, o2, np.full(512, np.nan)])[None, :, None, None, :]
    pl = np.array([l1, l2, -np.inf])[None, :, None, None]
    po = np.where(np.isnan(po), 0.0, po)
    o, l = combine_fp64(po, pl)
    ref = (math.exp(l1) * o1 + math.exp(l2) * o2) / (math.exp(l1) + math.exp(l2))
    assert np.allclose(o[0, 0, 0], ref, rtol=0, atol=1e-14)
    assert abs(l[0, 0, 0] - math.log(math.exp(l1) + math.exp(l2))) < 1e-14
    o, l = combine_fp64(np.zeros((1, 2, 1, 1, 512)), np.full((1, 2, 1, 1), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_empty_chunk_partial_is_minus_inf():
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=1, Sq=1, H=2, L=(64,))
    po, pl = split_partials_fp64(q8, qs, pool, ks, table, lens, P, SM, [[(0, 64), (64, 64)]])
    assert np.all(pl[0, 1] == -np.inf) and np.all(po[0, 1] == 0)


# ------------------------------------------ per-request query counts (ragged verify)

def test_per_request_query_counts_by_hand():
    """4 query slots; request 0 has 2 tokens over a 3-position context, request 1 none,
    request 2 all 4.  Request 0's token 0 sees positions 0-1 and token 1 sees 0-2 (written
    out with loops below); its slots 2 and 3, and all of request 1, see nothing."""
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=3, Sq=4, H=2, L=(3, 9, 40), seed=5)
    qlen = np.array([2, 0, 4], np.int32)
    o, lse = attention_fp64(q8, qs, pool, ks, table, lens, P, SM, q_lens=qlen)
    k = decode_e4m3(kv8[0]) * float(ks)
    for t, visible in ((0, 2), (1, 3)):
        for h in range(2):
            qd = decode_e4m3(q8[0, t, h]) * float(qs)
            z = [SM * sum(qd[d] * k[n, d] for d in range(576)) for n in range(visible)]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            ref = [sum(w[n] * k[n, c] for n in range(visible)) / sum(w) for c in range(512)]
            assert np.allclose(o[0, t, h], ref, rtol=0, atol=1e-12)
            assert abs(lse[0, t, h] - (m + math.log(sum(w)))) <= 1e-12
    assert np.all(o[0, 2:] == 0) and np.all(lse[0, 2:] == -np.inf)
    assert np.all(o[1] == 0) and np.all(lse[1] == -np.inf)
    full_o, full_l = attention_fp64(q8, qs, pool, ks, table, lens, P, SM, requests=[2])
    assert np.array_equal(o[2], full_o[0]) and np.array_equal(lse[2], full_l[0])


def test_full_query_counts_change_nothing():
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=2, Sq=3, H=4, L=(130, 4), seed=6)
    a = attention_fp64(q8, qs, pool, ks, table, lens, P, SM)
    b = attention_fp64(q8, qs, pool, ks, table, lens, P, SM, q_lens=[3, 3])
    c = attention_fp64(q8, qs, pool, ks, table, lens, P, SM, q_lens=[7, 99])   # clamped
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_short_request_is_the_same_as_a_call_with_fewer_slots():
    """A request with k of Sq tokens: its first k slots equal a call whose q8 holds only
    those k slots (the causal window shifts with k, not with Sq)."""
    q8, qs, kv8, ks, pool, table, P, lens = _rand_case(B=1, Sq=8, H=2, L=(300,), seed=7)
    for k in (1, 3, 5):
        o, lse = attention_fp64(q8, qs, pool, ks, table, lens, P, SM, q_lens=[k])
        o2, lse2 = attention_fp64(np.ascontiguousarray(q8[:, :k]), qs, pool, ks, table, lens, P,
                                  SM)
        assert np.array_equal(o[:, :k], o2) and np.array_equal(lse[:, :k], lse2)
        assert np.all(lse[:, k:] == -np.inf)
