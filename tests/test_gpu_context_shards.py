"""Context-parallel sharding of one request, shown on one GPU (runs on an MI355X).

A request's KV is cut into G contiguous shards, as G GPUs would hold it; each shard is
decoded on its own.  Either every shard's split partials go into its slice of one partial
buffer and one combine merges all G x S_local of them, or (what the GPUs would exchange)
each shard first merges its own splits into one partial row per query row
(mla_splitkv_combine_partial) and the final combine runs over the G merged partials.
The result must meet the oracle's contract for the whole request and agree with the
unsharded decode.  With several query tokens, the shards other than the last are told how
many context positions follow them (ctx_after), so that only the last one masks.
"""
import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from fp8_mla_split_amd.workload import materialize
from synthetic import WORKLOADS, Workload
from tests import oracle_side as ors
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


def _two_level(dw, G, S_local, batched_stride=True):
    """Each shard: decode, then merge its own splits into slice g of a [1, G, R] buffer (the
    rows an all-gather over G GPUs would assemble); then the combine over the G slices."""
    w = dw.w
    L = int(dw.seq_lens_host[0])
    Ls = L // G
    shards = dw.kv_pool8[0, :L].view(G, Ls, 576)
    R = w.heads
    po = torch.empty((1, S_local, R, 512), dtype=torch.float16, device="cuda")
    pl = torch.empty((1, S_local, R), dtype=torch.float32, device="cuda")
    go = torch.full((1, G, R, 512), float("nan"), dtype=torch.float16, device="cuda")
    gl = torch.full((1, G, R), float("nan"), dtype=torch.float32, device="cuda")
    lens = torch.full((1,), Ls, dtype=torch.int32, device="cuda")
    for g in range(G):
        table = torch.full((1, 1), g, dtype=torch.int32, device="cuda")
        mla.decode_splitkv(dw.q8, shards, table, lens, dw.q_scale, dw.kv_scale, w.softmax_scale,
                           Ls, S_local, 0, po, pl)
        mla.splitkv_combine_partial(po, pl, 1, R, go[:, g], gl[:, g], G * R)
    out, lse = mla.splitkv_combine(go, gl, 1, R, dw.kv_scale)
    torch.cuda.synchronize()
    return _bf16(out), lse.cpu().numpy(), go, gl


@pytest.mark.parametrize("G,S_local", [(2, 64), (8, 32), (8, 16)])
def test_two_level_merge_matches_the_oracle(b1, G, S_local):
    o, l, go, gl = _two_level(b1, G, S_local)
    assert torch.isfinite(gl).all() and torch.isfinite(go.float()).all()   # every slice written
    _compare(b1, o, l, _oracle(b1, [0]))
    flat_o, flat_l = _sharded(b1, G, S_local)
    assert np.max(np.abs(o - flat_o)) <= 2e-3
    assert np.max(np.abs(l - flat_l)) <= 1e-4


def test_partial_merge_of_a_plain_decode_equals_its_combine():
    """Batch 3 with an output stride: the merged partial, scaled by the KV scale and rounded
    to bf16, is the plain combine's output; its lse is the plain combine's lse."""
    w = Workload("merge_partial", batch=3, heads=32, q_tokens=2, context=None,
                 context_range=(1, 1), page_size=64, permuted_pool=True, seed=51)
    dw = materialize(w, seq_lens=np.array([300, 5000, 64], np.int32))
    po, pl, S = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                                   dw.kv_scale, w.softmax_scale, dw.max_seq_len, 7, 0)
    R = 64
    mo = torch.full((3, 2, R, 512), float("nan"), dtype=torch.float16, device="cuda")
    ml = torch.full((3, 2, R), float("nan"), dtype=torch.float32, device="cuda")
    mla.splitkv_combine_partial(po, pl, 2, 32, mo[:, 1], ml[:, 1], 2 * R)   # slice 1 of 2
    out, lse = mla.splitkv_combine(po, pl, 2, 32, dw.kv_scale)
    torch.cuda.synchronize()
    assert torch.isnan(ml[:, 0]).all() and torch.isnan(mo[:, 0].float()).all()   # untouched
    assert torch.allclose(ml[:, 1].reshape(3, 2, 32), lse, rtol=0, atol=1e-5)
    # the plain output is the same value rounded to bf16 (half an ulp: up to 2^-8 relative,
    # just above a power of two) where the partial holds it in fp16 (2^-11): within 2^-7
    scaled = (mo[:, 1].float() * dw.kv_scale).reshape(3, 2, 32, 512)
    assert torch.allclose(scaled, out.float(), rtol=2.0 ** -7, atol=1e-6)
    # merging a single merged partial again: the same value through one more rounding
    o2, l2 = mla.splitkv_combine(mo[:, 1:2].contiguous(), ml[:, 1:2].contiguous(), 2, 32,
                                 dw.kv_scale)
    torch.cuda.synchronize()
    assert torch.allclose(o2.float(), out.float(), rtol=2.0 ** -6, atol=1e-6)
    assert torch.equal(l2, ml[:, 1].reshape(3, 2, 32))
    _compare(dw, _bf16(o2), l2.cpu().numpy(), _oracle(dw, [0, 1, 2]))


@pytest.mark.parametrize("q_lens", [None, [8, 3]])
def test_shards_with_several_query_tokens(q_lens):
    """Verify shape (8 query tokens, causal among them) over 3 context shards per request:
    the shards other than the last are told how many positions follow them (ctx_after), so
    all their positions are visible; the last shard masks as usual.  Each shard's splits are
    merged into its slice, and the combine over the slices meets the oracle's contract for
    the whole requests (optionally with per-request draft counts)."""
    G, Ls, B, Sq, H = 3, 1024, 2, 8, 32
    w = Workload("cp_verify", batch=B, heads=H, q_tokens=Sq, context=G * Ls, seed=61)
    dw = materialize(w)
    R = Sq * H
    shards = dw.kv_pool8[:, :G * Ls].reshape(B * G, Ls, 576)   # page b * G + g
    po = torch.empty((B, 4, R, 512), dtype=torch.float16, device="cuda")
    pl = torch.empty((B, 4, R), dtype=torch.float32, device="cuda")
    go = torch.full((B, G, R, 512), float("nan"), dtype=torch.float16, device="cuda")
    gl = torch.full((B, G, R), float("nan"), dtype=torch.float32, device="cuda")
    lens = torch.full((B,), Ls, dtype=torch.int32, device="cuda")
    ql = None if q_lens is None else torch.tensor(q_lens, dtype=torch.int32, device="cuda")
    for g in range(G):
        table = (torch.arange(B, dtype=torch.int32, device="cuda") * G + g)[:, None].contiguous()
        after = torch.full((B,), (G - 1 - g) * Ls, dtype=torch.int32, device="cuda")
        mla.decode_splitkv(dw.q8, shards, table, lens, dw.q_scale, dw.kv_scale,
                           w.softmax_scale, Ls, 4, 0, po, pl, q_lens=ql, ctx_after=after)
        mla.splitkv_combine_partial(po, pl, Sq, H, go[:, g], gl[:, g], G * R)
    out, lse = mla.splitkv_combine(go, gl, Sq, H, dw.kv_scale)
    torch.cuda.synchronize()
    o, l = _bf16(out), lse.cpu().numpy()
    if q_lens is None:
        _compare(dw, o, l, _oracle(dw, range(B)))
        return
    q_scale, kv_scale = ors.scales(w, dw.seq_lens_host)
    for b in range(B):
        L = int(dw.seq_lens_host[b])
        ref_o, ref_l = ors.attention_request(w, b, L, ors.q8_request(w, b, q_scale), q_scale,
                                             ors.kv8_request(w, b, L, kv_scale), kv_scale,
                                             q_len=q_lens[b])
        k = q_lens[b]
        assert np.all(o[b][k:] == 0) and np.all(l[b][k:] == -np.inf)
        ors.check_output(o[b][:k], ref_o[:k], l[b][:k], ref_l[:k])


@pytest.mark.parametrize("Sq,H", [(1, 32), (8, 16)], ids=["sq1", "sq8"])
def test_uneven_shards_with_positions_after(Sq, H):
    """Shards whose lengths are not multiples of the 32-token tile (1000, 100 and 1300
    positions), each decoded in a padded buffer whose rows past the shard hold NaN bytes.
    Every shard but the last is told how many positions follow it (ctx_after), which lifts
    the causal limit past the shard's own end: positions past the shard must still count as
    absent (not as zero rows).  Two-level merge, compared with the oracle over the whole
    requests."""
    lens_g = [1000, 100, 1300]
    G, B = len(lens_g), 2
    w = Workload("cp_uneven", batch=B, heads=H, q_tokens=Sq, context=sum(lens_g), seed=71)
    dw = materialize(w)
    R = Sq * H
    go = torch.full((B, G, R, 512), float("nan"), dtype=torch.float16, device="cuda")
    gl = torch.full((B, G, R), float("nan"), dtype=torch.float32, device="cuda")
    off = 0
    for g, Ls in enumerate(lens_g):
        P = -(-Ls // 32) * 32
        shard = torch.full((B, P, 576), 0x7F, dtype=torch.uint8, device="cuda")
        shard[:, :Ls] = dw.kv_pool8[:, off:off + Ls]
        table = torch.arange(B, dtype=torch.int32, device="cuda")[:, None].contiguous()
        lens = torch.full((B,), Ls, dtype=torch.int32, device="cuda")
        after = torch.full((B,), sum(lens_g[g + 1:]), dtype=torch.int32, device="cuda")
        po, pl, _ = mla.decode_splitkv(dw.q8, shard, table, lens, dw.q_scale, dw.kv_scale,
                                       w.softmax_scale, Ls, 3, 0, ctx_after=after)
        mla.splitkv_combine_partial(po, pl, Sq, H, go[:, g], gl[:, g], G * R)
        off += Ls
    out, lse = mla.splitkv_combine(go, gl, Sq, H, dw.kv_scale)
    torch.cuda.synchronize()
    _compare(dw, _bf16(out), lse.cpu().numpy(), _oracle(dw, range(B)))
