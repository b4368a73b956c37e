"""C-ABI checks that need no GPU: exports, argument validation, planner (CPU only).

Every argument check in libmla.so runs before any HIP call, so invalid calls are rejected
here with fake (never dereferenced) device pointers.
"""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "fp8_mla_split_amd", "libmla.so")
HDR = os.path.join(ROOT, "include", "mla.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x1000)  # non-null, never dereferenced by a rejected call


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmla.so is not built (python -m fp8_mla_split_amd.build)")
    L = ctypes.CDLL(LIB)
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_quantize_fp8_sat.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_float, ctypes.c_void_p]
    i, f, v, i64 = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64
    L.mla_decode_splitkv.argtypes = [v, v, v, v, i, i, i, i, i, i, f, f, f, i, i, v, v, i64, v]
    L.mla_splitkv_combine.argtypes = [v, v, i, i, i, i, f, v, v, v]
    L.mla_splitkv_plan.argtypes = [i, i, i, i, i64, i, ctypes.POINTER(i), ctypes.POINTER(i),
                                   ctypes.POINTER(i64)]
    L.mla_decode_splitkv_dev_scales.argtypes = [v, v, v, v, i, i, i, i, i, i, v, v, f, i, i, v,
                                                v, i64, v]
    L.mla_splitkv_combine_dev_scale.argtypes = [v, v, i, i, i, i, v, v, v, v]
    L.mla_splitkv_combine_partial.argtypes = [v, v, i, i, i, i, v, v, i64, v]
    L.mla_decode_splitkv_ex.argtypes = [v, v, v, v, v, v, v, i, i, i, i, i, i, f, f, v, v, f, i,
                                        i, v, v, i64, v]
    L.mla_quantize_fp8_sat_dynamic.argtypes = [v, i, v, i64, v, v, i64, v]
    L.mla_kv_append_fp8_sat.argtypes = [v, i, v, i64, v, v, i, i, i, i, f, v]
    L.mla_decode_noalloc.argtypes = [v, v, v, v, i, i, i, i, i, i, f, f, f, i, v, v, v]
    L.mla_kv_append_rope_fp8_sat.argtypes = [v, i, v, i64, v, v, i, i, i, i, f, v, v, i64, v]
    return L


def header_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("mla_quantize_fp8_sat", "mla_decode_splitkv", "mla_splitkv_combine",
              "mla_splitkv_plan", "mla_status_string", "mla_quantize_fp8_sat_dynamic",
              "mla_kv_append_fp8_sat", "mla_decode_splitkv_dev_scales",
              "mla_splitkv_combine_dev_scale", "mla_decode_splitkv_ex",
              "mla_splitkv_combine_partial"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in header_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in [(0, b"MLA_OK"), (1, b"MLA_ERR_INVALID_ARG"), (2, b"MLA_ERR_UNSUPPORTED"),
                       (3, b"MLA_ERR_WORKSPACE"), (4, b"MLA_ERR_HIP"), (99, b"MLA_ERR_UNKNOWN")]:
        assert lib.mla_status_string(code) == name


def test_quantize_rejects_bad_arguments(lib):
    q = lib.mla_quantize_fp8_sat
    assert q(FAKE, FAKE, -1, 1.0, None) == INVALID
    assert q(FAKE, FAKE, 10, float("nan"), None) == INVALID
    assert q(FAKE, FAKE, 10, float("inf"), None) == INVALID
    assert q(FAKE, FAKE, 10, 0.0, None) == INVALID
    assert q(FAKE, FAKE, 10, -2.0, None) == INVALID
    assert q(None, FAKE, 10, 1.0, None) == INVALID
    assert q(FAKE, None, 10, 1.0, None) == INVALID
    assert q(None, None, 0, 1.0, None) == OK          # empty: nothing enqueued


def _decode(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, pt=FAKE, sl=FAKE, B=1, Sq=1, H=16, P=64, maxp=4, maxl=256,
             qs=1.0, ks=1.0, sm=0.07, S=4, r=128, po=FAKE, pl=FAKE, cap=1 << 20)
    a.update(kw)
    return lib.mla_decode_splitkv(a["q"], a["kv"], a["pt"], a["sl"], a["B"], a["Sq"], a["H"],
                                  a["P"], a["maxp"], a["maxl"], a["qs"], a["ks"], a["sm"],
                                  a["S"], a["r"], a["po"], a["pl"], a["cap"], None)


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, kv=None) == INVALID
    assert _decode(lib, pt=None) == INVALID
    assert _decode(lib, sl=None) == INVALID
    assert _decode(lib, po=None) == INVALID
    assert _decode(lib, pl=None) == INVALID
    assert _decode(lib, B=-1) == INVALID
    assert _decode(lib, Sq=0) == INVALID
    assert _decode(lib, H=0) == INVALID
    assert _decode(lib, maxp=0) == INVALID
    assert _decode(lib, S=-1) == INVALID
    assert _decode(lib, qs=float("nan")) == INVALID
    assert _decode(lib, ks=0.0) == INVALID
    assert _decode(lib, sm=float("inf")) == INVALID
    assert _decode(lib, cap=-1) == INVALID
    assert _decode(lib, S=0, maxl=0) == INVALID        # planner needs a length bound


def test_decode_unsupported_shapes_and_workspace(lib):
    assert _decode(lib, P=48) == UNSUPPORTED            # pages must hold whole 32-token tiles
    assert _decode(lib, P=16) == UNSUPPORTED
    assert _decode(lib, Sq=2, H=40000) == UNSUPPORTED   # more than 65536 rows
    assert _decode(lib, r=48) == UNSUPPORTED
    assert _decode(lib, r=32) == UNSUPPORTED
    assert _decode(lib, r=64) == UNSUPPORTED
    assert _decode(lib, S=70000) == UNSUPPORTED
    assert _decode(lib, cap=4 * 16 - 1) == WORKSPACE    # B*S*Sq*H = 64 entries needed
    assert _decode(lib, B=0, q=None, kv=None) == OK     # empty batch: nothing enqueued


def test_combine_rejects_bad_arguments(lib):
    c = lib.mla_splitkv_combine
    assert c(None, FAKE, 1, 4, 1, 16, 1.0, FAKE, None, None) == INVALID
    assert c(FAKE, None, 1, 4, 1, 16, 1.0, FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, 1.0, None, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 0, 1, 16, 1.0, FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, -1, 4, 1, 16, 1.0, FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, 0.0, FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, float("nan"), FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 5000, 1, 16, 1.0, FAKE, None, None) == UNSUPPORTED
    assert c(None, None, 0, 4, 1, 16, 1.0, None, None, None) == OK


def test_dynamic_quantize_rejects_bad_arguments(lib):
    q = lib.mla_quantize_fp8_sat_dynamic
    W = 4096
    assert q(FAKE, 0, FAKE, -1, FAKE, FAKE, W, None) == INVALID
    assert q(FAKE, 2, FAKE, 10, FAKE, FAKE, W, None) == INVALID        # unknown source type
    assert q(None, 0, FAKE, 10, FAKE, FAKE, W, None) == INVALID
    assert q(FAKE, 0, None, 10, FAKE, FAKE, W, None) == INVALID
    assert q(FAKE, 0, FAKE, 10, None, FAKE, W, None) == INVALID
    assert q(FAKE, 0, FAKE, 10, FAKE, None, W, None) == INVALID
    assert q(ctypes.c_void_p(0x1002), 0, FAKE, 10, FAKE, FAKE, W, None) == INVALID  # fp32 align
    assert q(ctypes.c_void_p(0x1001), 1, FAKE, 10, FAKE, FAKE, W, None) == INVALID  # bf16 align
    assert q(FAKE, 0, FAKE, 10, ctypes.c_void_p(0x1001), FAKE, W, None) == INVALID
    assert q(FAKE, 0, FAKE, 10, FAKE, FAKE, W - 1, None) == WORKSPACE
    assert q(None, 0, None, 0, None, None, 0, None) == OK                # empty: nothing enqueued


def test_kv_append_rejects_bad_arguments(lib):
    def a(src, pool, num_pages, pt, sl, B, T, P, maxp, scale, dtype=0):
        return lib.mla_kv_append_fp8_sat(src, dtype, pool, num_pages, pt, sl, B, T, P, maxp,
                                         scale, None)
    assert a(FAKE, FAKE, 8, FAKE, FAKE, -1, 1, 64, 4, 1.0) == INVALID
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, -1, 64, 4, 1.0) == INVALID
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, 1, 0, 4, 1.0) == INVALID
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, 1, 64, 0, 1.0) == INVALID
    assert a(FAKE, FAKE, 0, FAKE, FAKE, 2, 1, 64, 4, 1.0) == INVALID
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, 1, 64, 4, 0.0) == INVALID
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, 1, 64, 4, float("inf")) == INVALID
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, 1, 64, 4, 1.0, dtype=2) == INVALID   # unknown dtype
    for k in range(4):
        ptrs = [FAKE] * 4
        ptrs[k] = None
        assert a(ptrs[0], ptrs[1], 8, ptrs[2], ptrs[3], 2, 1, 64, 4, 1.0) == INVALID
    assert a(ctypes.c_void_p(0x1002), FAKE, 8, FAKE, FAKE, 2, 1, 64, 4, 1.0) == INVALID
    assert a(ctypes.c_void_p(0x1001), FAKE, 8, FAKE, FAKE, 2, 1, 64, 4, 1.0,
             dtype=1) == INVALID                                               # bf16 alignment
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 1 << 16, 1 << 16, 64, 4, 1.0) == UNSUPPORTED
    assert a(FAKE, FAKE, 8, FAKE, FAKE, 2, 1, 1 << 16, 1 << 16, 1.0) == UNSUPPORTED
    assert a(None, None, 8, None, None, 0, 1, 64, 4, 1.0) == OK    # empty batch
    assert a(None, None, 8, None, None, 2, 0, 64, 4, 1.0) == OK    # no new tokens


def test_dev_scale_variants_reject_bad_arguments(lib):
    d = lib.mla_decode_splitkv_dev_scales

    def dec(qs=FAKE, ks=FAKE, sm=0.07, **kw):
        a = dict(q=FAKE, B=1, P=64, cap=1 << 20)
        a.update(kw)
        return d(a["q"], FAKE, FAKE, FAKE, a["B"], 1, 16, a["P"], 4, 256, qs, ks, sm, 4, 128,
                 FAKE, FAKE, a["cap"], None)
    assert dec(qs=None) == INVALID
    assert dec(ks=None) == INVALID
    assert dec(qs=ctypes.c_void_p(0x1002)) == INVALID
    assert dec(sm=0.0) == INVALID
    assert dec(q=None) == INVALID
    assert dec(P=48) == UNSUPPORTED
    assert dec(cap=63) == WORKSPACE
    assert dec(B=0, q=None) == OK
    c = lib.mla_splitkv_combine_dev_scale
    assert c(FAKE, FAKE, 1, 4, 1, 16, None, FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, ctypes.c_void_p(0x1001), FAKE, None, None) == INVALID
    assert c(None, FAKE, 1, 4, 1, 16, FAKE, FAKE, None, None) == INVALID
    assert c(FAKE, FAKE, 1, 5000, 1, 16, FAKE, FAKE, None, None) == UNSUPPORTED
    assert c(None, None, 0, 4, 1, 16, FAKE, None, None, None) == OK


def test_decode_ex_rejects_bad_arguments(lib):
    d = lib.mla_decode_splitkv_ex

    def dec(ql=FAKE, ca=None, od=None, qsd=None, ksd=None, qs=1.0, ks=1.0, **kw):
        a = dict(q=FAKE, B=1, P=64, cap=1 << 20, Sq=8)
        a.update(kw)
        return d(a["q"], FAKE, FAKE, FAKE, ql, ca, od, a["B"], a["Sq"], 16, a["P"], 4, 256, qs,
                 ks, qsd, ksd, 0.07, 4, 128, FAKE, FAKE, a["cap"], None)
    assert dec(qsd=FAKE) == INVALID                     # one scale pointer without the other
    assert dec(ksd=FAKE) == INVALID
    assert dec(ql=ctypes.c_void_p(0x1002)) == INVALID   # q_lens misaligned
    assert dec(ca=ctypes.c_void_p(0x1001)) == INVALID   # ctx_after misaligned
    assert dec(od=ctypes.c_void_p(0x1003)) == INVALID   # order misaligned
    assert dec(qs=0.0) == INVALID                       # host scales checked when used
    # with device scales the host values are not used: the call gets as far as the
    # workspace check (which fails here, so nothing is launched)
    assert dec(qs=0.0, qsd=FAKE, ksd=FAKE, cap=8 * 16 * 4 - 1) == WORKSPACE
    assert dec(q=None) == INVALID
    assert dec(P=48) == UNSUPPORTED
    assert dec(cap=8 * 16 * 4 - 1) == WORKSPACE
    assert dec(B=0, q=None) == OK
    assert dec(B=0, q=None, ql=None) == OK


def test_combine_partial_rejects_bad_arguments(lib):
    c = lib.mla_splitkv_combine_partial
    assert c(None, FAKE, 1, 4, 1, 16, FAKE, FAKE, 16, None) == INVALID
    assert c(FAKE, None, 1, 4, 1, 16, FAKE, FAKE, 16, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, None, FAKE, 16, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, FAKE, None, 16, None) == INVALID   # lse is required
    assert c(FAKE, FAKE, 1, 0, 1, 16, FAKE, FAKE, 16, None) == INVALID
    assert c(FAKE, FAKE, 1, 4, 1, 16, FAKE, FAKE, 15, None) == INVALID   # stride < Sq*H
    assert c(FAKE, FAKE, 1, 5000, 1, 16, FAKE, FAKE, 16, None) == UNSUPPORTED
    assert c(None, None, 0, 4, 1, 16, None, None, 16, None) == OK


def _plan(lib, B, Sq, H, L, cu, total=0):
    s, r, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    st = lib.mla_splitkv_plan(B, Sq, H, L, total, cu, ctypes.byref(s), ctypes.byref(r),
                              ctypes.byref(n))
    return st, s.value, r.value, n.value


def test_plan_rejects_bad_arguments(lib):
    assert _plan(lib, 0, 1, 128, 1000, 256)[0] == INVALID
    assert _plan(lib, 1, 1, 128, 0, 256)[0] == INVALID
    assert _plan(lib, 1, 1, 128, 1000, -1)[0] == INVALID
    assert _plan(lib, 1, 2, 40000, 1000, 256)[0] == UNSUPPORTED
    assert _plan(lib, 2, 1, 128, 1000, 256, total=-1)[0] == INVALID
    assert _plan(lib, 2, 1, 128, 1000, 256, total=2001)[0] == INVALID   # > batch * max


@pytest.mark.parametrize("B,Sq,H,L", [(1, 1, 128, 131072), (16, 1, 128, 131072),
                                      (32, 1, 128, 131072), (4, 8, 128, 1048576),
                                      (1, 1, 16, 256), (3, 2, 48, 5000)])
def test_plan_fills_the_machine_and_is_consistent(lib, B, Sq, H, L):
    st, S, r, n = _plan(lib, B, Sq, H, L, 256)
    assert st == OK and S >= 1 and r == 128
    assert n == B * S * Sq * H
    G = -(-(Sq * H) // r)
    tiles = -(-L // 32)
    assert S <= max(1, tiles)                     # no more chunks than tiles
    if tiles >= 4 * 256:                          # long contexts: enough workgroups for 256 CUs
        assert B * S * G >= 256


def test_split_count_follows_cu_count_and_context(lib):
    """The split count is derived from the machine and the shape, not a constant."""
    s_256 = _plan(lib, 1, 1, 128, 131072, 256)[1]
    s_128 = _plan(lib, 1, 1, 128, 131072, 128)[1]
    s_short = _plan(lib, 1, 1, 128, 4096, 256)[1]
    assert s_128 < s_256
    assert s_short < s_256
    assert _plan(lib, 64, 1, 128, 131072, 256)[1] < s_256


def test_plan_total_tokens(lib):
    """Equal lengths: giving the total changes nothing.  Mixed lengths (the total well below
    batch x the longest): more splits, so the longest request's chunks shrink toward the
    average work per CU."""
    for B, L in [(1, 131072), (16, 131072), (32, 131072), (4, 1048576)]:
        assert _plan(lib, B, 1, 128, L, 256, total=B * L)[1:] == _plan(lib, B, 1, 128, L, 256)[1:]
    s_eq = _plan(lib, 32, 1, 128, 131072, 256)[1]
    s_mixed = _plan(lib, 32, 1, 128, 131072, 256, total=32 * 67584)[1]   # U[4K, 128K] mean
    assert s_mixed > s_eq


def test_graft_entry_build_imports_the_binding_in_a_fresh_process():
    """build() compiles and then imports the binding; the import half runs here in a fresh
    interpreter (the compile itself is replaced by a no-op so the test stays fast)."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import fp8_mla_split_amd.build as b\n"
        "b.build = lambda verbose=False: b.LIB\n"
        "import __graft_entry__ as g\n"
        "g.build(); g.build()\n"
        "import fp8_mla_split_amd as m\n"
        "assert m.status_string(0) == 'MLA_OK'\n" % ROOT
    )
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]


def test_read_probe_rejects_bad_arguments(lib):
    r = lib.mla_hbm_read_probe
    r.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert r(None, 32768, FAKE, 1, None) == INVALID
    assert r(FAKE, 32768, None, 1, None) == INVALID
    assert r(FAKE, 32768, FAKE, 0, None) == INVALID
    assert r(FAKE, 1000, FAKE, 1, None) == INVALID       # not a multiple of 32 KiB
    assert r(ctypes.c_void_p(0x1004), 32768, FAKE, 1, None) == INVALID  # not 16-byte aligned
    assert r(FAKE, 0, FAKE, 1, None) == OK                # nothing to read


def header_prototypes():
    """{name: [parameter declarations]} of every function the header declares, whitespace
    normalised."""
    text = re.sub(r"/\*.*?\*/", "", open(HDR).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\((.*?)\)\s*;", text,
                         flags=re.M | re.S):
        params = [" ".join(p.split()) for p in m.group(2).split(",")]
        protos[m.group(1)] = [p.replace(" *", "*").replace("* ", "*") for p in params]
    return protos


# The boundary as built, for the calls the path is made of.  It departs from the first
# proposal of the interface in these places, each for a stated reason:
#   - partial_o is fp16 (uint16_t bit patterns) in units of the KV scale, not fp32: it halves
#     the partials' traffic, and every value lies in [-448, 448];
#   - rows_per_group (query rows per workgroup) replaces a head-group count: a workgroup
#     holds rows of several query tokens when a request has fewer than 128 heads;
#   - partial_rows / partial_rows_capacity (entries of the partial buffers) replace a byte
#     count: the two buffers have different element sizes;
#   - the decode takes max_seq_len (the planner's input when num_splits is 0), the planner
#     takes total_kv_tokens (mixed lengths) and the combine v_scale (fp16 partials are in
#     KV-scale units);
#   - streams are void* (a hipStream_t), so the header needs no HIP include.
BOUNDARY = {
    "mla_quantize_fp8_sat": ["const float*src_dev", "uint8_t*dst_dev", "int64_t n",
                             "float scale", "void*stream"],
    "mla_splitkv_plan": ["int batch", "int q_tokens", "int heads", "int max_seq_len",
                         "int64_t total_kv_tokens", "int cu_count", "int*num_splits",
                         "int*rows_per_group", "int64_t*partial_rows"],
    "mla_decode_splitkv": ["const uint8_t*q8_dev", "const uint8_t*kv_pool_dev",
                           "const int32_t*page_table_dev", "const int32_t*seq_lens_dev",
                           "int batch", "int q_tokens", "int heads", "int page_size",
                           "int max_pages", "int max_seq_len", "float q_scale",
                           "float kv_scale", "float softmax_scale", "int num_splits",
                           "int rows_per_group", "uint16_t*partial_o_dev",
                           "float*partial_lse_dev", "int64_t partial_rows_capacity",
                           "void*stream"],
    "mla_splitkv_combine": ["const uint16_t*partial_o_dev", "const float*partial_lse_dev",
                            "int batch", "int num_splits", "int q_tokens", "int heads",
                            "float v_scale", "uint16_t*out_bf16_dev", "float*out_lse_dev",
                            "void*stream"],
    "mla_status_string": ["mla_status s"],
}


def test_boundary_prototypes_are_the_documented_ones():
    protos = header_prototypes()
    for name, params in BOUNDARY.items():
        assert protos.get(name) == params, (name, protos.get(name))


def test_decode_noalloc_rejects_bad_arguments(lib):
    d = lib.mla_decode_noalloc
    rows = (40 * 1024 * 1024 - 256) // 1028        # partial rows the library's array holds

    def dec(B=1, H=16, S=4, out=FAKE, q=FAKE, qs=1.0, P=64):
        return d(q, FAKE, FAKE, FAKE, B, 1, H, P, 4, 256, qs, 1.0, 0.07, S, out, None, None)
    assert dec(out=None) == INVALID
    assert dec(q=None) == INVALID
    assert dec(qs=0.0) == INVALID
    assert dec(P=48) == UNSUPPORTED
    assert dec(B=0, q=None, out=None) == OK                   # nothing to do
    assert dec(H=128, S=rows // 128 + 1) == WORKSPACE         # that many splits do not fit
    assert dec(B=rows // 128 + 1, H=128, S=0) == WORKSPACE    # not even one split fits


def test_kv_append_rope_rejects_bad_arguments(lib):
    def a(cos=FAKE, sin=FAKE, npos=100, B=2, T=1, src=FAKE, scale=1.0):
        return lib.mla_kv_append_rope_fp8_sat(src, 0, FAKE, 8, FAKE, FAKE, B, T, 64, 4, scale,
                                              cos, sin, npos, None)
    assert a(cos=None) == INVALID
    assert a(sin=None) == INVALID
    assert a(cos=ctypes.c_void_p(0x1002)) == INVALID          # tables 4-byte aligned
    assert a(npos=0) == INVALID
    assert a(scale=0.0) == INVALID                            # the append's own checks
    assert a(src=None) == INVALID
    assert a(B=0, cos=None, sin=None) == OK                   # nothing to write


def test_readme_c_example_compiles_against_the_header(tmp_path):
    """The README's example of one decode step is valid C against include/mla.h."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    text = open(os.path.join(ROOT, "README.md")).read()
    body = re.search(r"```c\n(.*?)```", text, flags=re.S).group(1)
    src = tmp_path / "example.c"
    src.write_text(
        '#include "mla.h"\n'
        "void example(int B, int Sq, int H, int max_len, const float* q_f32, uint8_t* q8,\n"
        "             float q_scale, void* stream, const void* new_kv, uint8_t* pool,\n"
        "             int64_t n_pages, const int32_t* table, const int32_t* lens, int max_pages,\n"
        "             float kv_scale, float softmax_scale, uint16_t* partial_o,\n"
        "             float* partial_lse, uint16_t* out_bf16, float* out_lse) {\n"
        + body + "}\n")
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-I",
                        os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
