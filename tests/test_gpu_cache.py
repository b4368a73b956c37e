"""GPU cache preparation vs the oracle (runs on an MI355X): the paged KV append and the
quantisation with a data-derived scale are bit-exact; the decode and combine that read their
scales on the device give the same bits as the host-scale calls, and match the oracle.
"""
import numpy as np
import pytest
import torch

import fp8_mla_split_amd as mla
from fp8_mla_split_amd.workload import materialize
from oracle import (append_kv_fp8, append_kv_rope_fp8, bf16_bits_to_f32, dynamic_quantize,
                    quantize_e4m3_sat)
from synthetic import WORKLOADS, Workload, q_f32
from tests import oracle_side as ors
from tests.test_gpu_decode import _bf16, _compare, _oracle

pytestmark = pytest.mark.gpu


# ------------------------------------------------------- data-derived scale

def _dyn_gpu(x: np.ndarray, bf16: bool = False, offset: int = 0):
    """GPU codes and scale for x (fp32 values, or bf16 bit patterns when bf16), placed
    `offset` elements into a larger buffer so that alignment can be varied."""
    if bf16:
        buf = torch.zeros(x.size + offset, dtype=torch.int16)
        buf[offset:] = torch.from_numpy(x.view(np.int16))
        t = buf.cuda().view(torch.bfloat16)[offset:]
    else:
        buf = torch.zeros(x.size + offset, dtype=torch.float32)
        buf[offset:] = torch.from_numpy(x)
        t = buf.cuda()[offset:]
    codes, scale = mla.quantize_fp8_sat_dynamic(t)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), np.float32(scale.cpu().numpy()[0])


SIZES = [1, 3, 17, 4096 + 5, 73_728, 1_000_037, (1 << 21) + 19]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1])
def test_dynamic_fp32_bit_exact(n, offset):
    rng = np.random.default_rng(n + offset)
    x = (rng.standard_normal(n) * rng.choice([1e-3, 1.0, 300.0])).astype(np.float32)
    codes, s = _dyn_gpu(x, offset=offset)
    ref, ref_s = dynamic_quantize(x)
    assert s == ref_s
    assert np.array_equal(codes, ref)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1])
def test_dynamic_bf16_bit_exact(n, offset):
    rng = np.random.default_rng(10 * n + offset)
    bits = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    # finite patterns only here (exponent field below all ones)
    bits = np.where((bits & 0x7F80) == 0x7F80, bits & 0xBFFF, bits).astype(np.uint16)
    codes, s = _dyn_gpu(bits, bf16=True, offset=offset)
    ref, ref_s = dynamic_quantize(bits, source="bf16")
    assert s == ref_s
    assert np.array_equal(codes, ref)


def test_dynamic_zeros_and_nan():
    codes, s = _dyn_gpu(np.zeros(1000, np.float32))
    assert s == 1.0 and not codes.any()
    x = np.random.default_rng(2).standard_normal(5000).astype(np.float32)
    x[1234] = np.nan
    codes, s = _dyn_gpu(x)
    assert np.isnan(s)
    assert np.all((codes & 0x7F) == 0x7F)


def test_dynamic_q_of_every_workload_matches_the_host_scale_path():
    """One step's Q at every workload's shape (the Q the decode reads): the data-derived
    scale equals the host's and the codes equal the oracle's."""
    for name in ("tiny", "b1_128k", "b16_128k", "verify_b4_1m"):
        q = q_f32(WORKLOADS[name])
        codes, s = _dyn_gpu(q.reshape(-1))
        ref, ref_s = dynamic_quantize(q.reshape(-1))
        assert s == ref_s, name
        assert np.array_equal(codes, ref), name


# ------------------------------------------------------------- KV append

def _append_case(rng, lens, t_new, page_size, max_pages, bad_page_req=None):
    B = len(lens)
    num_pages = B * max_pages + 3
    table = rng.permutation(num_pages)[:B * max_pages].astype(np.int32).reshape(B, max_pages)
    if bad_page_req is not None:
        table[bad_page_req, :] = -1
    pool = rng.integers(0, 256, size=(num_pages, page_size, 576), dtype=np.uint8)
    new = (rng.standard_normal((B, t_new, 576)) * 2.0).astype(np.float32)
    new[rng.random(new.shape) < 0.01] *= 1000.0            # saturating values
    return pool, table, np.asarray(lens, np.int32), new


@pytest.mark.parametrize("t_new,page_size", [(1, 64), (3, 32), (8, 64), (5, 96)])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_append_bit_exact(t_new, page_size, offset, src):
    rng = np.random.default_rng(100 * t_new + page_size + offset)
    max_pages = 6
    cap = max_pages * page_size
    # ordinary, shorter than T (leading rows skipped), exactly full, past the table, page -1
    lens = [100, max(t_new - 2, 0), cap, cap + 2, 50]
    pool, table, seq, new = _append_case(rng, lens, t_new, page_size, max_pages,
                                         bad_page_req=4)
    s = np.float32(2.0 * 4.5 / 448)
    g_pool = torch.from_numpy(pool).cuda()
    if src == "bf16":  # the rows as bf16 patterns (truncated), widened exactly by the oracle
        bits = (new.view(np.uint32) >> 16).astype(np.uint16)
        ref = append_kv_fp8(pool, table, seq, bf16_bits_to_f32(bits), s)
        buf = torch.zeros(new.size + offset, dtype=torch.int16)
        buf[offset:] = torch.from_numpy(bits.reshape(-1).view(np.int16))
        g_new = buf.cuda().view(torch.bfloat16)[offset:].view(new.shape)
    else:
        ref = append_kv_fp8(pool, table, seq, new, s)
        buf = torch.zeros(new.size + offset, dtype=torch.float32)
        buf[offset:] = torch.from_numpy(new.reshape(-1))
        g_new = buf.cuda()[offset:].view(new.shape)
    mla.kv_append_fp8_sat(g_new, g_pool, torch.from_numpy(table).cuda(),
                          torch.from_numpy(seq).cuda(), float(s))
    torch.cuda.synchronize()
    got = g_pool.cpu().numpy()
    assert np.array_equal(got, ref)


def _rope_tables(rng, positions, kind):
    if kind == "standard":  # theta_i = 10000^(-2i/64), angle n theta_i
        theta = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)
        ang = np.arange(positions)[:, None] * theta[None, :]
    else:
        ang = rng.uniform(-np.pi, np.pi, (positions, 32))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@pytest.mark.parametrize("t_new,page_size", [(1, 64), (8, 64), (5, 96)])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("tables", ["standard", "random", "random_unaligned"])
def test_append_rope_bit_exact(t_new, page_size, offset, src, tables):
    """RoPE fused with the append against the oracle: the rotated rope pairs and the plain
    latent columns, quantised, at every new row's position; rows whose position is past the
    angle tables, past the page table or on a page -1 are not written.  The vector path
    (16-byte aligned rows and tables) and the per-column path (offset rows or tables)."""
    rng = np.random.default_rng(7 * t_new + page_size + offset + len(tables))
    max_pages = 6
    cap = max_pages * page_size
    lens = [100, max(t_new - 2, 0), cap, cap + 2, 50, 300]
    pool, table, seq, new = _append_case(rng, lens, t_new, page_size, max_pages,
                                         bad_page_req=4)
    positions = 299                  # request 5's last position (299) is past the tables
    cos_t, sin_t = _rope_tables(rng, positions, "standard" if tables == "standard" else "random")
    s = np.float32(2.0 * 4.5 / 448)
    g_pool = torch.from_numpy(pool).cuda()
    if src == "bf16":
        bits = (new.view(np.uint32) >> 16).astype(np.uint16)
        ref = append_kv_rope_fp8(pool, table, seq, bf16_bits_to_f32(bits), s, cos_t, sin_t)
        buf = torch.zeros(new.size + offset, dtype=torch.int16)
        buf[offset:] = torch.from_numpy(bits.reshape(-1).view(np.int16))
        g_new = buf.cuda().view(torch.bfloat16)[offset:].view(new.shape)
    else:
        ref = append_kv_rope_fp8(pool, table, seq, new, s, cos_t, sin_t)
        buf = torch.zeros(new.size + offset, dtype=torch.float32)
        buf[offset:] = torch.from_numpy(new.reshape(-1))
        g_new = buf.cuda()[offset:].view(new.shape)
    if tables == "random_unaligned":   # tables at a 4-byte (not 16-byte) aligned address
        cbuf = torch.zeros(cos_t.size + 1, dtype=torch.float32, device="cuda")
        sbuf = torch.zeros(sin_t.size + 1, dtype=torch.float32, device="cuda")
        cbuf[1:] = torch.from_numpy(cos_t.reshape(-1)).cuda()
        sbuf[1:] = torch.from_numpy(sin_t.reshape(-1)).cuda()
        g_cos, g_sin = cbuf[1:].view(positions, 32), sbuf[1:].view(positions, 32)
    else:
        g_cos, g_sin = torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda()
    mla.kv_append_rope_fp8_sat(g_new, g_pool, torch.from_numpy(table).cuda(),
                               torch.from_numpy(seq).cuda(), float(s), g_cos, g_sin)
    torch.cuda.synchronize()
    got = g_pool.cpu().numpy()
    assert np.array_equal(got, ref)
    # and the rope columns really moved: the rotated rows differ from a plain append
    plain = append_kv_fp8(pool, table, seq, new if src == "f32" else bf16_bits_to_f32(bits), s)
    assert not np.array_equal(ref[..., 512:], plain[..., 512:])


def _append_sweep_cases(n=30, seed=20261206):
    """Append shapes drawn once: page sizes that are not multiples of the 32-token tile (1, 7,
    100, 333) beside the usual ones, 1-9 new rows per request, lengths below T, exactly at the
    table's end and past it, page ids outside the pool, fp32 or bf16 rows, with or without
    RoPE (tables that may end before some positions)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 6))
        T = int(rng.integers(1, 10))
        P = int(rng.choice([1, 7, 32, 64, 100, 333]))
        max_pages = int(rng.integers(1, 9))
        cap = max_pages * P
        lens = [int(rng.choice([rng.integers(0, cap + 1), cap, cap + int(rng.integers(1, 5)),
                                max(T - int(rng.integers(1, 3)), 0)])) for _ in range(B)]
        bad = int(rng.integers(0, B)) if rng.random() < 0.4 else None
        src = "bf16" if rng.random() < 0.4 else "f32"
        rope = rng.random() < 0.5
        positions = int(rng.integers(1, cap + 5)) if rope else 0
        out.append((f"a{i:02d}_b{B}_t{T}_p{P}_m{max_pages}_{src}" + ("_rope" if rope else ""),
                    B, T, P, max_pages, lens, bad, src, positions, int(rng.integers(0, 1 << 30))))
    return out


APPEND_SWEEP = _append_sweep_cases()


@pytest.mark.parametrize("case", APPEND_SWEEP, ids=[c[0] for c in APPEND_SWEEP])
def test_append_sweep_bit_exact(case):
    name, B, T, P, max_pages, lens, bad, src, positions, seed = case
    print(f"[append] {name} lens {lens} bad page request {bad} rope positions {positions}",
          flush=True)
    rng = np.random.default_rng(seed)
    pool, table, seq, new = _append_case(rng, lens, T, P, max_pages, bad_page_req=bad)
    s = np.float32(2.0 * 4.5 / 448)
    if src == "bf16":
        bits = (new.view(np.uint32) >> 16).astype(np.uint16)
        rows = bf16_bits_to_f32(bits)
        g_new = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        rows = new
        g_new = torch.from_numpy(new).cuda()
    g_pool = torch.from_numpy(pool).cuda()
    g_table, g_seq = torch.from_numpy(table).cuda(), torch.from_numpy(seq).cuda()
    if positions:
        cos_t, sin_t = _rope_tables(rng, positions, "random")
        ref = append_kv_rope_fp8(pool, table, seq, rows, s, cos_t, sin_t)
        mla.kv_append_rope_fp8_sat(g_new, g_pool, g_table, g_seq, float(s),
                                   torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda())
    else:
        ref = append_kv_fp8(pool, table, seq, rows, s)
        mla.kv_append_fp8_sat(g_new, g_pool, g_table, g_seq, float(s))
    torch.cuda.synchronize()
    assert np.array_equal(g_pool.cpu().numpy(), ref)


def test_append_then_decode_reads_the_new_rows():
    """Step-by-step: a request's last 3 rows are appended (one step at a time) into a cache
    whose first rows came from the plain quantiser; the decode over the result matches the
    oracle over the whole quantised request."""
    w = Workload("append_decode", batch=2, heads=32, q_tokens=1, context=None,
                 context_range=(1, 1), page_size=64, permuted_pool=True, seed=9)
    lens = np.array([700, 1290], np.int32)
    dw = materialize(w, seq_lens=lens, keep_f32=True)
    # overwrite the last 3 rows of every request with NaN bytes, then append them back
    pool_host = dw.kv_pool8.cpu().numpy()
    for b, L in enumerate(lens):
        for n in range(L - 3, L):
            pool_host[dw.page_table_host[b, n // 64], n % 64] = 0x7F
    dw.kv_pool8.copy_(torch.from_numpy(pool_host))
    for k in range(3):
        step_lens = torch.from_numpy(lens - 2 + k).cuda()
        rows = torch.stack([dw.kv_f32[b][int(lens[b]) - 3 + k] for b in range(2)])[:, None]
        mla.kv_append_fp8_sat(rows.contiguous(), dw.kv_pool8, dw.page_table, step_lens,
                              dw.kv_scale)
    po, pl, _ = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                                   dw.kv_scale, w.softmax_scale, dw.max_seq_len, 3, 0)
    out, lse = mla.splitkv_combine(po, pl, 1, 32, dw.kv_scale)
    torch.cuda.synchronize()
    _compare(dw, _bf16(out), lse.cpu().numpy(), _oracle(dw, [0, 1]))


def test_append_at_paged_workload_size():
    """The paged workload's cache (1.25 GB, 32 requests): one new row per request whose last
    page has room, at its next position; requests without room are given a length past
    their page table and must be skipped.  The new rows equal the oracle's codes and the rest
    of every touched page is unchanged."""
    w = WORKLOADS["paged_b32"]
    dw = materialize(w)
    P = w.page_size
    lens = dw.seq_lens_host.astype(np.int64)
    room = lens % P != 0
    assert room.sum() >= 8
    past = dw.page_table_host.shape[1] * P + 1
    new_lens = np.where(room, lens + 1, past).astype(np.int32)
    rng = np.random.default_rng(11)
    new = (rng.standard_normal((w.batch, 1, 576)) * 3.0).astype(np.float32)
    pages = [int(dw.page_table_host[b, (lens[b] - 1) // P]) for b in range(w.batch)]
    before = dw.kv_pool8[pages].cpu().numpy()
    mla.kv_append_fp8_sat(torch.from_numpy(new).cuda(), dw.kv_pool8, dw.page_table,
                          torch.from_numpy(new_lens).cuda(), dw.kv_scale)
    torch.cuda.synchronize()
    after = dw.kv_pool8[pages].cpu().numpy()
    expect = before.copy()
    for b in range(w.batch):
        if room[b]:
            expect[b, lens[b] % P] = quantize_e4m3_sat(new[b, 0], np.float32(dw.kv_scale))
    assert np.array_equal(after, expect)


# ------------------------------------------------- scales kept on the device

def _run_dev(dw, q_scale_t, kv_scale_t, S):
    po, pl, S = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, q_scale_t,
                                   kv_scale_t, dw.w.softmax_scale, dw.max_seq_len, S, 0)
    out, lse = mla.splitkv_combine(po, pl, dw.w.q_tokens, dw.w.heads, kv_scale_t)
    torch.cuda.synchronize()
    return po.cpu().numpy(), pl.cpu().numpy(), _bf16(out), lse.cpu().numpy()


def _run_host(dw, S):
    po, pl, S = mla.decode_splitkv(dw.q8, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.q_scale,
                                   dw.kv_scale, dw.w.softmax_scale, dw.max_seq_len, S, 0)
    out, lse = mla.splitkv_combine(po, pl, dw.w.q_tokens, dw.w.heads, dw.kv_scale)
    torch.cuda.synchronize()
    return po.cpu().numpy(), pl.cpu().numpy(), _bf16(out), lse.cpu().numpy()


@pytest.mark.parametrize("name,S", [("tiny", 4), ("b1_128k", 0), ("b1_128k", 64)])
def test_dynamic_q_scale_decode_matches_host_path_and_oracle(name, S):
    """Q quantised with its scale derived on the device, decode and combine reading the
    scales on the device: the same bits as the host-scale calls (which the oracle pins), and
    within the contract of the oracle on the tiny workload."""
    w = WORKLOADS[name]
    dw = materialize(w)
    q8_dyn, qs_dev = mla.quantize_fp8_sat_dynamic(torch.from_numpy(q_f32(w)).cuda())
    torch.cuda.synchronize()
    assert np.float32(qs_dev.item()) == np.float32(dw.q_scale)
    assert torch.equal(q8_dyn, dw.q8)
    ks_dev = torch.tensor([dw.kv_scale], dtype=torch.float32, device="cuda")
    got = _run_dev(dw, qs_dev, ks_dev, S)
    ref = _run_host(dw, S)
    assert np.array_equal(got[0].view(np.uint16), ref[0].view(np.uint16))   # partial O
    assert np.array_equal(got[1], ref[1])                                  # partial lse
    assert np.array_equal(got[2], ref[2]) and np.array_equal(got[3], ref[3])
    if name == "tiny":
        _compare(dw, got[2], got[3], _oracle(dw, [0]))


def test_dev_scales_on_paged_causal_case():
    w = Workload("dev_paged", batch=3, heads=32, q_tokens=8, context=None, context_range=(1, 1),
                 page_size=64, permuted_pool=True, seed=21)
    dw = materialize(w, seq_lens=np.array([8, 300, 1029], np.int32))
    qs = torch.tensor([dw.q_scale], dtype=torch.float32, device="cuda")
    ks = torch.tensor([dw.kv_scale], dtype=torch.float32, device="cuda")
    got, ref = _run_dev(dw, qs, ks, 4), _run_host(dw, 4)
    assert np.array_equal(got[0].view(np.uint16), ref[0].view(np.uint16))
    assert np.array_equal(got[2], ref[2]) and np.array_equal(got[3], ref[3])
    _compare(dw, got[2], got[3], _oracle(dw, [0, 1, 2]))


def test_device_scale_step_replays_in_a_graph():
    """Append + Q amax/quantise + device-scale decode + combine captured in one HIP graph:
    every replay (with eager work and synchronisations between replays) gives the eager
    result bit for bit; nothing in the chain needs clearing before a replay."""
    w = Workload("graph_dev", batch=2, heads=64, q_tokens=1, context=None, context_range=(1, 1),
                 page_size=64, permuted_pool=True, seed=41)
    lens = np.array([1500, 2100], np.int32)
    dw = materialize(w, seq_lens=lens, keep_f32=True)
    q32 = torch.from_numpy(q_f32(w)).cuda()
    last = torch.stack([dw.kv_f32[b][int(lens[b]) - 1] for b in range(2)])[:, None].contiguous()
    ks = torch.tensor([dw.kv_scale], dtype=torch.float32, device="cuda")
    q8 = torch.empty(q32.shape, dtype=torch.uint8, device="cuda")
    qs = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(mla.QUANTIZE_DYNAMIC_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
    S = 5
    po = torch.empty((2, S, 64, 512), dtype=torch.float16, device="cuda")
    pl = torch.empty((2, S, 64), dtype=torch.float32, device="cuda")
    out = torch.empty((2, 1, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 1, 64), dtype=torch.float32, device="cuda")

    def step():
        mla.kv_append_fp8_sat(last, dw.kv_pool8, dw.page_table, dw.seq_lens, dw.kv_scale)
        mla.quantize_fp8_sat_dynamic(q32, out=q8, scale=qs, workspace=ws)
        mla.decode_splitkv(q8, dw.kv_pool8, dw.page_table, dw.seq_lens, qs, ks, w.softmax_scale,
                           dw.max_seq_len, S, 0, po, pl)
        mla.splitkv_combine(po, pl, 1, 64, ks, out=out, out_lse=lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        qs.fill_(-1.0)
        ws.fill_(0x7FFFFFFF)                       # stale maxima must not leak into the scale
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), rep
        assert torch.equal(lse, ref_l), rep
        assert np.float32(qs.item()) == np.float32(dw.q_scale)
    _compare(dw, _bf16(out), lse.cpu().numpy(), _oracle(dw, [0, 1]))


def test_dynamic_quantize_past_one_grid_of_work():
    """More elements than one pass of the capped grid covers (8192 workgroups x 256 threads
    x 16 values, and 1024 workgroups for the maxima), with a ragged tail: every element is
    reached by the grid-stride loops and the maximum is the whole tensor's."""
    n = (1 << 25) + (1 << 20) + 37
    x = np.random.default_rng(12).standard_normal(n).astype(np.float32)
    x[n - 5] = 97.25                                            # the maximum sits in the tail
    codes, s = _dyn_gpu(x)
    assert s == np.float32(97.25) / np.float32(448)
    ref = quantize_e4m3_sat(x, s, threads=8)
    assert np.array_equal(codes, ref)


def test_append_many_rows_per_launch():
    """A bulk append (4 requests x 16384 new rows, 36 threads per row: more units than one
    grid of 8192 x 256 threads covers at once) into a permuted pool, against the oracle."""
    rng = np.random.default_rng(13)
    B, T, P, maxp = 4, 16384, 64, 272
    lens = np.array([16384, 17000, 17408, 16500], np.int32)
    pool, table, seq, new = _append_case(rng, list(lens), T, P, maxp)
    s = np.float32(0.013)
    ref = append_kv_fp8(pool, table, seq, new, s)
    g_pool = torch.from_numpy(pool).cuda()
    mla.kv_append_fp8_sat(torch.from_numpy(new).cuda(), g_pool, torch.from_numpy(table).cuda(),
                          torch.from_numpy(seq).cuda(), float(s))
    torch.cuda.synchronize()
    assert np.array_equal(g_pool.cpu().numpy(), ref)
