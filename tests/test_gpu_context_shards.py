"""Context-parallel sharding of one request, shown on one GPU (runs on an MI355X).

A request's KV is cut into G contiguous shards, as G GPUs would hold it; each shard is
decoded on its own into its slice of the split-partial buffer (the slices an all-gather
would assemble), and one combine over all G x S_local partials gives the request's output.
The result must meet the oracle's contract for the whole request and agree with the
unsharded decode.  Single query token per request (every shard's positions are visible to
it); for several query tokens only the last shard would need the causal mask.
"""
import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from fp8_mla_split_amd.workload import materialize
from synthetic import WORKLOADS
from tests.test_gpu_decode import _bf16, _compare, _oracle

pytestmark = pytest.mark.gpu


def _sharded(dw, G, S_local):
    w = dw.w
    L = int(dw.seq_lens_host[0])
    assert w.batch == 1 and w.q_tokens == 1 and L % (32 * G) == 0
    Ls = L // G
    shards = dw.kv_pool8[0, :L].view(G, Ls, 576)            # shard g = positions [g Ls, (g+1) Ls)
    rows = w.heads
    po = torch.empty((1, G * S_local, rows, 512), dtype=torch.float16, device="cuda")
    pl = torch.empty((1, G * S_local, rows), dtype=torch.float32, device="cuda")
    lens = torch.full((1,), Ls, dtype=torch.int32, device="cuda")
    for g in range(G):
        table = torch.full((1, 1), g, dtype=torch.int32, device="cuda")
        mla.decode_splitkv(dw.q8, shards, table, lens, dw.q_scale, dw.kv_scale, w.softmax_scale,
                           Ls, S_local, 0, po[:, g * S_local:(g + 1) * S_local],
                           pl[:, g * S_local:(g + 1) * S_local])
    out, lse = mla.splitkv_combine(po, pl, 1, w.heads, dw.kv_scale)
    torch.cuda.synchronize()
    return _bf16(out), lse.cpu().numpy()


@pytest.fixture(scope="module")
def b1():
    dw = materialize(WORKLOADS["b1_128k"])
    yield dw
    del dw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("G,S_local", [(2, 128), (4, 64), (8, 32), (8, 0)])
def test_shards_combine_to_the_whole_request(b1, G, S_local):
    if S_local == 0:  # what the planner picks for one shard
        S_local = mla.splitkv_plan(1, 1, 128, int(b1.seq_lens_host[0]) // G).num_splits
    o, l = _sharded(b1, G, S_local)
    _compare(b1, o, l, _oracle(b1, [0]))
    po, pl, _ = mla.decode_splitkv(b1.q8, b1.kv_pool8, b1.page_table, b1.seq_lens, b1.q_scale,
                                   b1.kv_scale, b1.w.softmax_scale, b1.max_seq_len,
                                   G * S_local, 0)
    ref, ref_l = mla.splitkv_combine(po, pl, 1, 128, b1.kv_scale)
    torch.cuda.synchronize()
    # another partition of the same sum: far inside the contract
    assert np.max(np.abs(o - _bf16(ref))) <= 2e-3
    assert np.max(np.abs(l - ref_l.cpu().numpy())) <= 1e-4
