"""mla_decode_noalloc against the two calls it stands for (runs on an MI355X).

The entry point runs the split-KV decode and the combine with the split partials in the
library's own device array, so the caller passes only inputs and outputs.  Its result must be
the one mla_decode_splitkv + mla_splitkv_combine give with the same split count, bit for bit
(same kernels, same partition), and it must meet the oracle's contract.  Two calls in a row,
the second with a smaller input: the array keeps the first call's contents, which the second
must not see.  A third shape needs its planned split count reduced so that the partials fit.
"""
import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from fp8_mla_split_amd.workload import materialize
from synthetic import Workload
from tests.test_gpu_decode import _bf16, _compare, _oracle

pytestmark = pytest.mark.gpu

ARRAY_ROWS = (40 * 1024 * 1024 - 256) // 1028   # partial rows (fp16 row + lse) the array holds


def _workload(name, B, H, Sq, lens, P, seed):
    w = Workload(name, batch=B, heads=H, q_tokens=Sq, context=None, context_range=(1, 1),
                 page_size=P, permuted_pool=P > 0, seed=seed)
    return materialize(w, seq_lens=np.array(lens, np.int32))


def _noalloc(dw, S):
    w = dw.w
    return mla.decode_noalloc(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                              dw.kv_scale, w.softmax_scale, dw.max_seq_len, S)


def _two_calls(dw, S):
    w = dw.w
    po, pl, _ = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                                   dw.kv_scale, w.softmax_scale, dw.max_seq_len, S, 0)
    return mla.splitkv_combine(po, pl, w.q_tokens, w.heads, dw.kv_scale)


def _same(a, b):
    (ao, al), (bo, bl) = a, b
    torch.cuda.synchronize()
    assert torch.equal(ao.view(torch.int16), bo.view(torch.int16))
    assert torch.equal(al, bl)


def test_two_calls_in_a_row_the_second_smaller():
    big = _workload("noalloc_big", 4, 128, 2, [9000, 20000, 3000, 12345], 64, 81)
    small = _workload("noalloc_small", 1, 16, 1, [300], 0, 82)
    for dw in (big, small):
        w = dw.w
        S = mla.splitkv_plan(w.batch, w.q_tokens, w.heads, dw.max_seq_len).num_splits
        assert w.batch * S * w.q_tokens * w.heads <= ARRAY_ROWS   # the planned count fits
        got = _noalloc(dw, 0)                                      # planner inside the call
        _same(got, _two_calls(dw, S))
        _compare(dw, _bf16(got[0]), got[1].cpu().numpy(), _oracle(dw, range(w.batch)))
        _same(_noalloc(dw, 3), _two_calls(dw, 3))                  # a given split count


def test_planned_split_count_reduced_to_fit():
    dw = _workload("noalloc_many", 200, 128, 1, [2048] * 200, 0, 83)
    w = dw.w
    planned = mla.splitkv_plan(w.batch, 1, w.heads, dw.max_seq_len).num_splits
    assert planned * w.batch * w.heads > ARRAY_ROWS >= w.batch * w.heads
    fit = ARRAY_ROWS // (w.batch * w.heads)
    got = _noalloc(dw, 0)
    _same(got, _two_calls(dw, min(planned, fit)))
    _compare(dw, _bf16(got[0]), got[1].cpu().numpy(), _oracle(dw, [0, 199]))
    with pytest.raises(mla.MLAError):                              # a given count that does not fit
        _noalloc(dw, fit + 1)


def test_captured_in_a_graph_and_replayed():
    """The use it is made for: the Q quantisation and the no-allocation decode captured into a
    HIP graph (nothing to allocate, no memset), replayed three times with other work and
    synchronisations in between; every replay equals the eager result bit for bit."""
    dw = _workload("noalloc_graph", 2, 128, 1, [20000, 7000], 64, 84)
    w = dw.w
    from synthetic import q_f32
    q32 = torch.from_numpy(q_f32(w)).cuda()
    q8 = torch.empty(q32.shape, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, 1, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, 1, w.heads), dtype=torch.float32, device="cuda")

    def step():
        mla.quantize_fp8_sat(q32, dw.q_scale, out=q8)
        mla.decode_noalloc(q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale, dw.kv_scale,
                           w.softmax_scale, dw.max_seq_len, 0, out=out, out_lse=lse)
    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    assert torch.equal(q8, dw.q8)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for k in range(3):
        out.zero_()
        lse.zero_()
        _noalloc(_workload(f"noalloc_between_{k}", 1, 16, 1, [500 + 100 * k], 0, 85 + k), 2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same((out, lse), ref)
