"""GPU split-KV decode + combine vs the fp64 oracle (runs on an MI355X).

Small cases cover several tiles, ragged tails, causal multi-token queries, paged pools with
NaN-poisoned page tails, row counts that do not fill a workgroup, and every row-group size.
The full-size workloads are checked on sampled requests and heads, in the launch
configuration the benchmark uses (planner's choice, plus the fixed 64-way split).
"""
import math
import zlib
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from fp8_mla_split_amd.workload import materialize
from oracle import quantize_e4m3_sat
from synthetic import WORKLOADS, Workload
from tests import oracle_side as ors

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(192.0)


def _bf16(t: torch.Tensor) -> np.ndarray:
    return ors.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def _run(dw, num_splits=0, rows_per_group=0):
    po, pl, S = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                                   dw.kv_scale, dw.w.softmax_scale, dw.max_seq_len,
                                   num_splits, rows_per_group)
    out, lse = mla.splitkv_combine(po, pl, dw.w.q_tokens, dw.w.heads, dw.kv_scale)
    torch.cuda.synchronize()
    return _bf16(out), lse.cpu().numpy(), S


def _oracle(dw, requests, heads=None):
    w = dw.w
    q_scale, kv_scale = ors.scales(w, dw.seq_lens_host)
    assert np.float32(dw.q_scale) == q_scale and np.float32(dw.kv_scale) == kv_scale
    res = {}
    for b in requests:
        L = int(dw.seq_lens_host[b])
        kv8 = ors.kv8_request(w, b, L, kv_scale)
        q8 = ors.q8_request(w, b, q_scale)
        res[b] = ors.attention_request(w, b, L, q8, q_scale, kv8, kv_scale, heads)
    return res


def _compare(dw, got_o, got_l, ref, heads=None):
    stats = []
    for b, (o_ref, l_ref) in ref.items():
        go = got_o[b] if heads is None else got_o[b][:, heads]
        gl = got_l[b] if heads is None else got_l[b][:, heads]
        stats.append(ors.check_output(go, o_ref, gl, l_ref))
    # measured errors of the sampled requests (shown with pytest -s)
    print(f"[parity] {dw.w.name}: requests {list(ref)} max abs "
          f"{max(s[0] for s in stats):.3e}, normalised L1 {max(s[1] for s in stats):.3e}")
    return stats


# ------------------------------------------------------------------ small cases

SMALL = [
    # name, B, H, Sq, lens, page_size, permuted, splits, rows_per_group
    ("one_token", 1, 16, 1, [1], 0, False, 1, 128),
    ("ragged_tail", 2, 16, 1, [33, 95], 0, False, 2, 128),
    ("several_tiles_h48", 1, 48, 1, [1000], 0, False, 3, 128),
    ("causal_sq2", 2, 16, 2, [2, 70], 0, False, 1, 128),
    ("causal_sq8_paged", 3, 32, 8, [8, 300, 129], 64, True, 4, 128),
    ("paged_p32", 4, 64, 1, [31, 64, 65, 2049], 32, True, 5, 128),
    ("rows_128", 1, 128, 1, [4500], 0, False, 8, 128),
    ("h256_rows64", 2, 256, 1, [700, 1300], 64, True, 3, 128),
    ("more_splits_than_tiles", 1, 16, 1, [100], 0, False, 16, 128),
    # pages of an odd number of 32-token tiles (steps straddle pages) and of several pairs
    ("paged_p96_odd_tiles", 2, 32, 1, [300, 1000], 96, True, 3, 128),
    ("paged_p128_causal", 2, 16, 4, [130, 1500], 128, True, 4, 128),
    # a chunk that is a single step, and chunks whose last step has one tile
    ("one_step_chunks", 1, 16, 1, [64 * 5], 0, False, 5, 128),
    ("odd_tile_tails", 2, 16, 1, [32 * 7, 32 * 9 + 5], 64, True, 2, 128),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_match_oracle(case):
    name, B, H, Sq, lens, P, perm, S, r = case
    w = Workload(name, batch=B, heads=H, q_tokens=Sq, context=None, context_range=(1, 1),
                 page_size=P, permuted_pool=perm, seed=zlib.crc32(name.encode()) % 1000)
    dw = materialize(w, seq_lens=np.array(lens, np.int32))
    o, l, _ = _run(dw, S, r)
    ref = _oracle(dw, range(B))
    _compare(dw, o, l, ref)


def test_empty_request_and_short_context():
    w = Workload("edge", batch=3, heads=16, q_tokens=4, context=None, context_range=(1, 1),
                 page_size=64, permuted_pool=True, seed=5)
    dw = materialize(w, seq_lens=np.array([0, 2, 80], np.int32))
    o, l, _ = _run(dw, 3, 128)
    assert np.all(o[0] == 0) and np.all(l[0] == -np.inf)       # nothing to attend to
    # L = 2 < Sq = 4: query tokens 0 and 1 see nothing, tokens 2 and 3 see 1 and 2 positions
    assert np.all(o[1][:2] == 0) and np.all(l[1][:2] == -np.inf)
    ref = _oracle(dw, [1, 2])
    ors.check_output(o[1][2:], ref[1][0][2:], l[1][2:], ref[1][1][2:])
    ors.check_output(o[2], ref[2][0], l[2], ref[2][1])


def test_repeat_runs_are_bitwise_identical():
    w = Workload("det", batch=2, heads=64, q_tokens=1, context=3000, page_size=64,
                 permuted_pool=True, seed=3)
    dw = materialize(w)
    a = _run(dw, 7, 128)
    b = _run(dw, 7, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_count_does_not_change_the_answer():
    w = Workload("splits", batch=1, heads=32, q_tokens=1, context=8192, seed=4)
    dw = materialize(w)
    ref = _oracle(dw, [0])
    outs = []
    for S, r in [(1, 128), (2, 128), (7, 128), (64, 128), (256, 128)]:
        o, l, _ = _run(dw, S, r)
        _compare(dw, o, l, ref)
        outs.append(o)
    # different partitions of the same sum agree far inside the contract
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2e-3


# ------------------------------------------------------------- full workloads

@pytest.fixture(scope="module")
def full():
    cache = {}

    def get(key):
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[key] = materialize(WORKLOADS[key])
        return cache[key]

    yield get
    cache.clear()
    torch.cuda.empty_cache()


def test_tiny_workload(full):
    dw = full("tiny")
    o, l, S = _run(dw, 4, 0)
    assert S == 4
    _compare(dw, o, l, _oracle(dw, [0]))


@pytest.mark.parametrize("splits", [64, 0])
def test_b1_128k(full, splits):
    dw = full("b1_128k")
    o, l, S = _run(dw, splits, 0)
    _compare(dw, o, l, _oracle(dw, [0]))


def test_b16_128k_sampled(full):
    dw = full("b16_128k")
    o, l, _ = _run(dw)
    _compare(dw, o, l, _oracle(dw, [0, 9, 15]))


@pytest.mark.parametrize("with_total", [False, True])
def test_paged_b32_sampled(full, with_total):
    """Planned inside the decode call (every request assumed as long as the longest), and as
    the benchmark plans it (the requests' total length given to the planner)."""
    dw = full("paged_b32")
    S = 0
    if with_total:
        w = dw.w
        S = mla.splitkv_plan(w.batch, w.q_tokens, w.heads, dw.max_seq_len,
                             total_kv_tokens=dw.kv_tokens).num_splits
    o, l, _ = _run(dw, S)
    lens = dw.seq_lens_host
    picks = [int(np.argmin(lens)), int(np.argmax(lens)), 13]
    _compare(dw, o, l, _oracle(dw, picks))


def test_verify_b4_1m_sampled(full):
    dw = full("verify_b4_1m")
    o, l, _ = _run(dw)
    heads = [0, 40, 77, 127]  # one head in each wave's 32 rows
    _compare(dw, o, l, _oracle(dw, [0, 3], heads=heads), heads=heads)


def _place(kv8_rows, lens, page_size, seed):
    """A pool holding the given per-request code rows: contiguous (page_size 0) or pages of
    page_size tokens in a random permutation; unused rows hold NaN bytes."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    if page_size == 0:
        P = max(64, -(-max(lens) // 64) * 64)
        table = np.arange(B, dtype=np.int32)[:, None]
        n_pages = B
    else:
        P = page_size
        npg = [-(-L // P) for L in lens]
        order = rng.permutation(int(sum(npg)))
        table = np.zeros((B, max(npg)), np.int32)
        off = 0
        for b, k in enumerate(npg):
            table[b, :k] = order[off:off + k]
            off += k
        n_pages = int(sum(npg))
    pool = torch.full((n_pages, P, 576), 0x7F, dtype=torch.uint8, device="cuda")
    flat = pool.view(-1, 576)
    for b, L in enumerate(lens):
        n = torch.arange(L, device="cuda")
        tb = torch.from_numpy(table[b].astype(np.int64)).cuda()
        flat[tb[n // P] * P + n % P] = kv8_rows[b]
    return pool, torch.from_numpy(table).cuda()


def test_output_is_bit_identical_across_layouts_and_batches():
    """The decode's arithmetic depends on a request's data and its chunk partition only, not
    on where its rows sit in memory or on what else is in the batch: contiguous, 64-token
    pages and 96-token pages (three tiles: the steps straddle pages) give the same bits, and
    so does a request decoded alone, in a batch, or dispatched in another order."""
    lens = [3000, 777, 5123]
    w = Workload("bitid", batch=3, heads=64, q_tokens=2, context=None, context_range=(1, 1),
                 page_size=0, seed=91)
    dw = materialize(w, seq_lens=np.array(lens, np.int32))
    rows = [dw.kv_pool8[b, :L] for b, L in enumerate(lens)]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    S, ml = 3, max(lens)

    def run(pool, table, q8, seq_lens, order=None):
        po, pl, _ = mla.decode_splitkv(q8, pool, table, seq_lens, dw.q_scale, dw.kv_scale,
                                       w.softmax_scale, ml, S, 0, order=order)
        out, lse = mla.splitkv_combine(po, pl, w.q_tokens, w.heads, dw.kv_scale)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu(), lse.cpu()

    ref = run(*_place(rows, lens, 0, 1), dw.q8, sl)
    for P in (64, 96, 128):
        got = run(*_place(rows, lens, P, P), dw.q8, sl)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), P
    order = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    got = run(*_place(rows, lens, 64, 7), dw.q8, sl, order=order)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    for b in range(3):   # alone, as a batch of one
        alone = run(*_place([rows[b]], [lens[b]], 64, 11 + b), dw.q8[b:b + 1].contiguous(),
                    sl[b:b + 1].contiguous())
        assert torch.equal(alone[0], ref[0][b:b + 1]) and torch.equal(alone[1], ref[1][b:b + 1])
    _compare(dw, _bf16(ref[0].view(torch.bfloat16).cuda()), ref[1].numpy(), _oracle(dw, [0, 1, 2]))
