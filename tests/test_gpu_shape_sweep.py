"""Seeded sweep of decode shapes against the fp64 oracle (runs on an MI355X).

Forty configurations drawn once from a fixed seed: batch 1-4, heads from 1 to 200, 1-8 query
tokens (causal among them), lengths from 0 to 3000 drawn per request (so one call mixes
empty, sub-tile, ragged and multi-chunk requests; at least one request per call is not
empty), contiguous or paged pools (page sizes of an odd and an even number of 32-token
tiles, permuted or in order), and the planner's split count or a fixed one from 1 to 40.
Every request and head is compared element by element with the oracle, to the same contract
as the named workloads.  A second sweep of 24 draws does the same through the per-request
path: draft counts from 0 to Sq per request (slots past a count must be O = 0, lse = -inf),
a random dispatch order in half of them and device-side scales in some.  A third, of 16
draws, cuts each request's context into 2-5 shards at random points (later shards of other
requests may be empty; rows past a shard hold NaN bytes), decodes every shard on its own with
the count of positions after it, merges each shard's splits into one partial row per query
row, and checks the final merge against the oracle over the whole requests.
"""
import zlib

import numpy as np
import pytest

from fp8_mla_split_amd.workload import materialize
from synthetic import Workload
from tests.test_gpu_decode import _compare, _oracle, _run

pytestmark = pytest.mark.gpu

HEADS = (1, 2, 8, 16, 24, 48, 64, 100, 128, 200)
PAGES = (0, 0, 32, 64, 96, 128, 256)


def _cases(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        H = int(rng.choice(HEADS))
        Sq = int(rng.integers(1, 9)) if rng.random() < 0.4 else 1
        while Sq * H > 512:
            Sq = max(1, Sq // 2)
        lens = rng.integers(0, 3001, size=B)
        lens[rng.random(B) < 0.15] = 0
        lens[rng.random(B) < 0.15] = rng.integers(1, 40)
        if lens.max() == 0:  # an all-empty batch is its own edge case (test_gpu_decode.py)
            lens[0] = 1 + (97 * i) % 3000
        P = int(rng.choice(PAGES))
        perm = bool(P and rng.random() < 0.7)
        S = 0 if rng.random() < 0.4 else int(rng.integers(1, 41))
        out.append((f"c{i:02d}_b{B}_h{H}_sq{Sq}_p{P}_s{S}", B, H, Sq, [int(x) for x in lens], P,
                    perm, S))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shape_sweep_matches_oracle(case):
    name, B, H, Sq, lens, P, perm, S = case
    print(f"[sweep] {name} lens {lens} permuted {perm}", flush=True)
    w = Workload(name, batch=B, heads=H, q_tokens=Sq, context=None, context_range=(1, 1),
                 page_size=P, permuted_pool=perm, seed=zlib.crc32(name.encode()) % 1000)
    dw = materialize(w, seq_lens=np.array(lens, np.int32))
    o, l, _ = _run(dw, S, 0)
    ref = _oracle(dw, range(B))
    _compare(dw, o, l, ref)


def _ragged_cases(n=24, seed=20261204):
    """Per-request draft counts (0..Sq), sometimes a dispatch order and device-side scales."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 6))
        H = int(rng.choice(HEADS))
        Sq = int(rng.integers(2, 9))
        while Sq * H > 512:
            Sq = max(2, Sq // 2)
        lens = rng.integers(1, 3001, size=B)
        lens[rng.random(B) < 0.2] = rng.integers(1, 12)
        q_lens = rng.integers(0, Sq + 1, size=B)
        P = int(rng.choice(PAGES))
        S = 0 if rng.random() < 0.4 else int(rng.integers(1, 33))
        order = rng.permutation(B) if rng.random() < 0.5 else None
        dev = bool(rng.random() < 0.3)
        out.append((f"r{i:02d}_b{B}_h{H}_sq{Sq}_p{P}_s{S}", B, H, Sq, [int(x) for x in lens],
                    [int(x) for x in q_lens], P, S,
                    None if order is None else [int(x) for x in order], dev))
    return out


RAGGED = _ragged_cases()


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged_sweep_matches_oracle(case):
    import torch

    import fp8_mla_split_amd as mla
    from tests.test_gpu_decode import _bf16
    from tests.test_gpu_verify_ragged import _check

    name, B, H, Sq, lens, q_lens, P, S, order, dev = case
    print(f"[sweep] {name} lens {lens} q_lens {q_lens} order {order} device scales {dev}",
          flush=True)
    w = Workload(name, batch=B, heads=H, q_tokens=Sq, context=None, context_range=(1, 1),
                 page_size=P, permuted_pool=bool(P), seed=zlib.crc32(name.encode()) % 1000)
    dw = materialize(w, seq_lens=np.array(lens, np.int32))
    if dev:
        qs = torch.tensor([dw.q_scale], dtype=torch.float32, device="cuda")
        ks = torch.tensor([dw.kv_scale], dtype=torch.float32, device="cuda")
    else:
        qs, ks = dw.q_scale, dw.kv_scale
    ql = torch.tensor(q_lens, dtype=torch.int32, device="cuda")
    od = None if order is None else torch.tensor(order, dtype=torch.int32, device="cuda")
    po, pl, _ = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, qs, ks,
                                   w.softmax_scale, dw.max_seq_len, S, 0, q_lens=ql, order=od)
    out, lse = mla.splitkv_combine(po, pl, Sq, H, ks)
    torch.cuda.synchronize()
    _check(dw, _bf16(out), lse.cpu().numpy(), q_lens, range(B))


def _shard_cases(n=16, seed=20261205):
    """Requests cut into 2-5 context shards at random points, each shard decoded on its own
    (as G GPUs would) and merged in two levels; sometimes with draft counts."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.choice(HEADS))
        Sq = int(rng.integers(1, 9)) if rng.random() < 0.5 else 1
        while Sq * H > 256:
            Sq = max(1, Sq // 2)
        G = int(rng.integers(2, 6))
        lens = rng.integers(G, 4001, size=B)
        cuts = []
        for L in lens:  # G shards of at least one position each (request 0), 0 allowed after
            lo = 1 if not cuts else 0
            inner = np.sort(rng.choice(np.arange(lo, int(L) - lo + 1), size=G - 1, replace=lo == 0))
            c = [0] + [int(x) for x in inner] + [int(L)]
            if lo and len(set(c)) < G + 1:  # shards of request 0 are never empty
                c = [int(round(k * int(L) / G)) for k in range(G + 1)]
            cuts.append(c)
        S = [int(x) for x in rng.integers(1, 9, size=G)]
        q_lens = [int(x) for x in rng.integers(0, Sq + 1, size=B)] if rng.random() < 0.4 else None
        out.append((f"g{i:02d}_b{B}_h{H}_sq{Sq}_G{G}", B, H, Sq, [int(x) for x in lens], cuts, S,
                    q_lens))
    return out


SHARDS = _shard_cases()


@pytest.mark.parametrize("case", SHARDS, ids=[c[0] for c in SHARDS])
def test_shard_sweep_matches_oracle(case):
    import torch

    import fp8_mla_split_amd as mla
    from tests import oracle_side as ors
    from tests.test_gpu_decode import _bf16
    from tests.test_gpu_verify_ragged import _check

    name, B, H, Sq, lens, cuts, S, q_lens = case
    G = len(S)
    print(f"[sweep] {name} lens {lens} cuts {cuts} splits {S} q_lens {q_lens}", flush=True)
    w = Workload(name, batch=B, heads=H, q_tokens=Sq, context=None, context_range=(1, 1),
                 seed=zlib.crc32(name.encode()) % 1000)
    dw = materialize(w, seq_lens=np.array(lens, np.int32))
    R = Sq * H
    go = torch.full((B, G, R, 512), float("nan"), dtype=torch.float16, device="cuda")
    gl = torch.full((B, G, R), float("nan"), dtype=torch.float32, device="cuda")
    ql = None if q_lens is None else torch.tensor(q_lens, dtype=torch.int32, device="cuda")
    table = torch.arange(B, dtype=torch.int32, device="cuda")[:, None].contiguous()
    for g in range(G):
        ls = [c[g + 1] - c[g] for c in cuts]
        P = max(32, -(-max(ls) // 32) * 32)
        shard = torch.full((B, P, 576), 0x7F, dtype=torch.uint8, device="cuda")  # NaN bytes
        for b in range(B):
            shard[b, :ls[b]] = dw.kv_pool8[b, cuts[b][g]:cuts[b][g + 1]]
        slen = torch.tensor(ls, dtype=torch.int32, device="cuda")
        after = torch.tensor([lens[b] - cuts[b][g + 1] for b in range(B)], dtype=torch.int32,
                             device="cuda")
        po, pl, _ = mla.decode_splitkv(dw.q8, shard, table, slen, dw.q_scale, dw.kv_scale,
                                       w.softmax_scale, max(ls), S[g], 0, q_lens=ql,
                                       ctx_after=after)
        mla.splitkv_combine_partial(po, pl, Sq, H, go[:, g], gl[:, g], G * R)
    out, lse = mla.splitkv_combine(go, gl, Sq, H, dw.kv_scale)
    torch.cuda.synchronize()
    o, l = _bf16(out), lse.cpu().numpy()
    _check(dw, o, l, q_lens if q_lens is not None else [Sq] * B, range(B))
