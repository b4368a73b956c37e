"""GPU verify step with a different number of query tokens per request (q_lens), against
the fp64 oracle (runs on an MI355X).  Slots past a request's count must come out as O = 0,
lse = -inf; with every count at its maximum the output is the plain call's, bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from fp8_mla_split_amd.workload import materialize
from synthetic import WORKLOADS, Workload
from tests import oracle_side as ors
from tests.test_gpu_decode import _bf16

pytestmark = pytest.mark.gpu


def _run(dw, q_lens, S, dev_scales=False):
    ql = None if q_lens is None else torch.from_numpy(np.asarray(q_lens, np.int32)).cuda()
    if dev_scales:
        qs = torch.tensor([dw.q_scale], dtype=torch.float32, device="cuda")
        ks = torch.tensor([dw.kv_scale], dtype=torch.float32, device="cuda")
    else:
        qs, ks = dw.q_scale, dw.kv_scale
    po, pl, _ = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, qs, ks,
                                   dw.w.softmax_scale, dw.max_seq_len, S, 0, q_lens=ql)
    out, lse = mla.splitkv_combine(po, pl, dw.w.q_tokens, dw.w.heads, ks)
    torch.cuda.synchronize()
    return _bf16(out), lse.cpu().numpy()


def _check(dw, o, l, q_lens, requests, heads=None):
    w = dw.w
    q_scale, kv_scale = ors.scales(w, dw.seq_lens_host)
    for b in requests:
        k = int(min(max(q_lens[b], 0), w.q_tokens))
        L = int(dw.seq_lens_host[b])
        ref_o, ref_l = ors.attention_request(w, b, L, ors.q8_request(w, b, q_scale), q_scale,
                                             ors.kv8_request(w, b, L, kv_scale), kv_scale,
                                             heads, q_len=k)
        go = o[b] if heads is None else o[b][:, heads]
        gl = l[b] if heads is None else l[b][:, heads]
        assert np.all(go[k:] == 0) and np.all(gl[k:] == -np.inf), b
        if k > 0:
            ors.check_output(go[:k], ref_o[:k], gl[:k], ref_l[:k])


CASES = [
    # name, B, H, Sq, lens, q_lens, page_size, splits
    ("mixed_p64", 4, 16, 8, [8, 300, 1029, 64], [8, 3, 1, 0], 64, 3),
    ("h128_row_groups", 3, 128, 8, [2000, 777, 64], [5, 8, 2], 64, 4),
    ("odd_tile_pages", 3, 32, 4, [130, 1500, 97], [2, 4, 1], 96, 5),
    ("counts_past_context", 2, 16, 8, [3, 40], [6, 8], 32, 2),   # fewer positions than tokens
    ("device_counts_clamped", 2, 16, 4, [500, 600], [-3, 99], 64, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ragged_counts_match_oracle(case):
    name, B, H, Sq, lens, q_lens, P, S = case
    w = Workload(name, batch=B, heads=H, q_tokens=Sq, context=None, context_range=(1, 1),
                 page_size=P, permuted_pool=True, seed=zlib.crc32(name.encode()) % 1000)
    dw = materialize(w, seq_lens=np.array(lens, np.int32))
    o, l = _run(dw, q_lens, S)
    _check(dw, o, l, q_lens, range(B))


def test_ragged_with_device_scales_is_bitwise_the_host_scale_result():
    w = Workload("ragged_dev", batch=3, heads=32, q_tokens=8, context=None, context_range=(1, 1),
                 page_size=64, permuted_pool=True, seed=31)
    dw = materialize(w, seq_lens=np.array([900, 64, 2048], np.int32))
    q_lens = [7, 1, 4]
    a = _run(dw, q_lens, 4)
    b = _run(dw, q_lens, 4, dev_scales=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    _check(dw, *a, q_lens, range(3))


def test_full_counts_equal_the_plain_call():
    w = Workload("ragged_full", batch=2, heads=64, q_tokens=8, context=3000, page_size=64,
                 permuted_pool=True, seed=32)
    dw = materialize(w)
    a = _run(dw, None, 5)
    b = _run(dw, [8, 8], 5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_verify_b4_1m_with_ragged_counts_sampled():
    """The speculative-verify workload (4 requests x 1M context, 8 slots) with 8, 5, 2 and 7
    draft tokens, in the planner's launch configuration; sampled requests and heads."""
    dw = materialize(WORKLOADS["verify_b4_1m"])
    q_lens = [8, 5, 2, 7]
    o, l = _run(dw, q_lens, 0)
    _check(dw, o, l, q_lens, [1, 2], heads=[0, 40, 77, 127])  # one head per wave
    for b in (0, 3):
        k = q_lens[b]
        assert np.all(o[b][k:] == 0) and np.all(l[b][k:] == -np.inf)


def test_dispatch_order_does_not_change_the_result():
    """Requests dispatched longest first (or in any permutation) give the same bits as
    request order: each workgroup's work does not depend on when it runs."""
    w = Workload("order", batch=5, heads=32, q_tokens=2, context=None, context_range=(1, 1),
                 page_size=64, permuted_pool=True, seed=71)
    dw = materialize(w, seq_lens=np.array([200, 5000, 64, 3000, 1200], np.int32))

    def run(order):
        od = None if order is None else torch.tensor(order, dtype=torch.int32, device="cuda")
        po, pl, _ = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens,
                                       dw.q_scale, dw.kv_scale, w.softmax_scale,
                                       dw.max_seq_len, 6, 0, order=od)
        out, lse = mla.splitkv_combine(po, pl, 2, 32, dw.kv_scale)
        torch.cuda.synchronize()
        return _bf16(out), lse.cpu().numpy()
    a = run(None)
    for order in ([1, 3, 4, 0, 2], [4, 3, 2, 1, 0]):
        b = run(order)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), order
    _check(dw, *a, [2] * 5, range(5))


def test_paged_b32_longest_first_sampled():
    """The paged workload dispatched longest first, planned with the requests' total length
    as the benchmark does: sampled requests against the oracle."""
    dw = materialize(WORKLOADS["paged_b32"])
    w = dw.w
    S = mla.splitkv_plan(w.batch, w.q_tokens, w.heads, dw.max_seq_len,
                         total_kv_tokens=dw.kv_tokens).num_splits
    order = torch.from_numpy(np.argsort(-dw.seq_lens_host, kind="stable").astype(np.int32))
    po, pl, _ = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                                   dw.kv_scale, w.softmax_scale, dw.max_seq_len, S, 0,
                                   order=order.cuda())
    out, lse = mla.splitkv_combine(po, pl, 1, w.heads, dw.kv_scale)
    torch.cuda.synchronize()
    lens = dw.seq_lens_host
    picks = [int(np.argmin(lens)), int(np.argmax(lens)), 13]
    _check(dw, _bf16(out), lse.cpu().numpy(), [1] * w.batch, picks)
