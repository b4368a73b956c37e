"""ctypes binding of libmla.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels.  PyTorch provides device memory
(``tensor.data_ptr()``) and the stream (``torch.cuda.current_stream()``); outputs that the
caller does not pass are allocated with torch.  Names follow ``include/mla.h``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmla.so")
if not os.path.exists(lib_path):
    raise ImportError(f"{lib_path} is not built; run `python -m fp8_mla_split_amd.build`")
_lib = ctypes.CDLL(lib_path)

_i32, _i64, _f32, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_status_string.argtypes = [_i32]
_lib.mla_quantize_fp8_sat.restype = _i32
_lib.mla_quantize_fp8_sat.argtypes = [_vp, _vp, _i64, _f32, _vp]
_lib.mla_splitkv_plan.restype = _i32
_lib.mla_splitkv_plan.argtypes = [_i32, _i32, _i32, _i32, _i64, _i32, ctypes.POINTER(_i32),
                                  ctypes.POINTER(_i32), ctypes.POINTER(_i64)]
_lib.mla_decode_splitkv.restype = _i32
_lib.mla_decode_splitkv.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _f32, _f32, _f32, _i32, _i32, _vp, _vp, _i64, _vp]
_lib.mla_splitkv_combine.restype = _i32
_lib.mla_splitkv_combine.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp]
_lib.mla_decode_splitkv_dev_scales.restype = _i32
_lib.mla_decode_splitkv_dev_scales.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _vp, _vp, _f32, _i32, _i32, _vp, _vp, _i64,
                                               _vp]
_lib.mla_decode_splitkv_ex.restype = _i32
_lib.mla_decode_splitkv_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _f32, _f32, _vp, _vp, _f32, _i32, _i32,
                                       _vp, _vp, _i64, _vp]
_lib.mla_splitkv_combine_partial.restype = _i32
_lib.mla_splitkv_combine_partial.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i64,
                                             _vp]
_lib.mla_splitkv_combine_dev_scale.restype = _i32
_lib.mla_splitkv_combine_dev_scale.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                               _vp]
_lib.mla_quantize_fp8_sat_dynamic.restype = _i32
_lib.mla_quantize_fp8_sat_dynamic.argtypes = [_vp, _i32, _vp, _i64, _vp, _vp, _i64, _vp]
_lib.mla_kv_append_fp8_sat.restype = _i32
_lib.mla_kv_append_fp8_sat.argtypes = [_vp, _i32, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _f32, _vp]
_lib.mla_decode_noalloc.restype = _i32
_lib.mla_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                    _f32, _f32, _i32, _vp, _vp, _vp]
_lib.mla_kv_append_rope_fp8_sat.restype = _i32
_lib.mla_kv_append_rope_fp8_sat.argtypes = [_vp, _i32, _vp, _i64, _vp, _vp, _i32, _i32, _i32,
                                            _i32, _f32, _vp, _vp, _i64, _vp]
_lib.mla_hbm_read_probe.restype = _i32
_lib.mla_hbm_read_probe.argtypes = [_vp, _i64, _vp, _i32, _vp]

D_KV, D_V = 576, 512
QUANTIZE_DYNAMIC_WORKSPACE_BYTES = 4096  # MLA_QUANTIZE_DYNAMIC_WORKSPACE_BYTES
_SRC_DTYPE = {torch.float32: 0, torch.bfloat16: 1}  # MLA_SRC_F32, MLA_SRC_BF16


class MLAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


def status_string(code: int) -> str:
    return _lib.mla_status_string(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != 0:
        raise MLAError(code, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev_tensor(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on the GPU")


@dataclass(frozen=True)
class Plan:
    num_splits: int
    rows_per_group: int
    partial_rows: int


def quantize_fp8_sat(x: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None):
    """e4m3 codes (uint8, same shape) of ``x / scale`` with saturation to +-448."""
    _dev_tensor(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _dev_tensor(out, torch.uint8, "out")
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _check(_lib.mla_quantize_fp8_sat(_ptr(x), _ptr(out), x.numel(), float(scale),
                                     _stream(x.device)), "mla_quantize_fp8_sat")
    return out


def quantize_fp8_sat_dynamic(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                             scale: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None):
    """Per-tensor scale amax / 448 taken on the device, then the saturating encode.

    x: fp32 or bf16 on the GPU.  Returns ``(codes uint8 [x.shape], scale fp32 [1])``; the
    scale stays on the device (pass it to decode_splitkv / splitkv_combine as is)."""
    if not x.is_cuda or x.dtype not in _SRC_DTYPE or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 or bf16 tensor on the GPU")
    dev = x.device
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(QUANTIZE_DYNAMIC_WORKSPACE_BYTES // 4, dtype=torch.int32,
                                device=dev)
    _dev_tensor(out, torch.uint8, "out")
    _dev_tensor(scale, torch.float32, "scale")
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _check(_lib.mla_quantize_fp8_sat_dynamic(
        _ptr(x), _SRC_DTYPE[x.dtype], _ptr(out), x.numel(), _ptr(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev)),
        "mla_quantize_fp8_sat_dynamic")
    return out, scale


def kv_append_fp8_sat(new_kv: torch.Tensor, kv_pool8: torch.Tensor, page_table: torch.Tensor,
                      seq_lens: torch.Tensor, kv_scale: float) -> None:
    """Quantise new_kv [B, T, 576] (fp32 or bf16) into the paged cache kv_pool8 [pages, P, 576]
    at positions seq_lens[b] - T + t (seq_lens already counts the new tokens)."""
    if not new_kv.is_cuda or new_kv.dtype not in _SRC_DTYPE or not new_kv.is_contiguous():
        raise ValueError("new_kv must be a contiguous fp32 or bf16 tensor on the GPU")
    _dev_tensor(kv_pool8, torch.uint8, "kv_pool8")
    _dev_tensor(page_table, torch.int32, "page_table")
    _dev_tensor(seq_lens, torch.int32, "seq_lens")
    if new_kv.dim() != 3 or new_kv.shape[2] != D_KV or kv_pool8.dim() != 3 or \
            kv_pool8.shape[2] != D_KV:
        raise ValueError("new_kv and kv_pool8 rows must be 576 wide")
    B, T = new_kv.shape[0], new_kv.shape[1]
    if page_table.dim() != 2 or page_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("page_table must be [B, max_pages] and seq_lens [B]")
    _check(_lib.mla_kv_append_fp8_sat(
        _ptr(new_kv), _SRC_DTYPE[new_kv.dtype], _ptr(kv_pool8), kv_pool8.shape[0],
        _ptr(page_table), _ptr(seq_lens), B, T,
        kv_pool8.shape[1], page_table.shape[1], float(kv_scale), _stream(new_kv.device)),
        "mla_kv_append_fp8_sat")


def kv_append_rope_fp8_sat(new_kv: torch.Tensor, kv_pool8: torch.Tensor, page_table: torch.Tensor,
                           seq_lens: torch.Tensor, kv_scale: float, rope_cos: torch.Tensor,
                           rope_sin: torch.Tensor) -> None:
    """kv_append_fp8_sat with each new row's rope pairs rotated first by the angle of its
    position: rope_cos / rope_sin are fp32 [positions, 32] tables on the GPU."""
    if not new_kv.is_cuda or new_kv.dtype not in _SRC_DTYPE or not new_kv.is_contiguous():
        raise ValueError("new_kv must be a contiguous fp32 or bf16 tensor on the GPU")
    _dev_tensor(kv_pool8, torch.uint8, "kv_pool8")
    _dev_tensor(page_table, torch.int32, "page_table")
    _dev_tensor(seq_lens, torch.int32, "seq_lens")
    _dev_tensor(rope_cos, torch.float32, "rope_cos")
    _dev_tensor(rope_sin, torch.float32, "rope_sin")
    if new_kv.dim() != 3 or new_kv.shape[2] != D_KV or kv_pool8.dim() != 3 or \
            kv_pool8.shape[2] != D_KV:
        raise ValueError("new_kv and kv_pool8 rows must be 576 wide")
    if rope_cos.dim() != 2 or rope_cos.shape[1] != 32 or rope_sin.shape != rope_cos.shape:
        raise ValueError("rope_cos and rope_sin must both be [positions, 32]")
    B, T = new_kv.shape[0], new_kv.shape[1]
    if page_table.dim() != 2 or page_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("page_table must be [B, max_pages] and seq_lens [B]")
    _check(_lib.mla_kv_append_rope_fp8_sat(
        _ptr(new_kv), _SRC_DTYPE[new_kv.dtype], _ptr(kv_pool8), kv_pool8.shape[0],
        _ptr(page_table), _ptr(seq_lens), B, T, kv_pool8.shape[1], page_table.shape[1],
        float(kv_scale), _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
        _stream(new_kv.device)), "mla_kv_append_rope_fp8_sat")


def _dev_scale(t, name: str) -> bool:
    """True for a device scale (a 1-element fp32 GPU tensor), False for a host number."""
    if isinstance(t, torch.Tensor):
        if not t.is_cuda or t.dtype != torch.float32 or t.numel() < 1:
            raise ValueError(f"{name} as a tensor must be fp32 on the GPU")
        return True
    return False


def splitkv_plan(batch: int, q_tokens: int, heads: int, max_seq_len: int,
                 cu_count: int = 0, total_kv_tokens: int = 0) -> Plan:
    """Split count and row grouping; total_kv_tokens = the sum of the requests' lengths if
    known (0: every request is max_seq_len long)."""
    s, r, n = _i32(), _i32(), _i64()
    _check(_lib.mla_splitkv_plan(batch, q_tokens, heads, max_seq_len, int(total_kv_tokens),
                                 cu_count,
                                 ctypes.byref(s), ctypes.byref(r), ctypes.byref(n)),
           "mla_splitkv_plan")
    return Plan(s.value, r.value, n.value)


def decode_splitkv(q8: torch.Tensor, kv_pool8: torch.Tensor, page_table: torch.Tensor,
                   seq_lens: torch.Tensor, q_scale: float, kv_scale: float,
                   softmax_scale: float, max_seq_len: int, num_splits: int = 0,
                   rows_per_group: int = 0, partial_o: Optional[torch.Tensor] = None,
                   partial_lse: Optional[torch.Tensor] = None,
                   q_lens: Optional[torch.Tensor] = None,
                   ctx_after: Optional[torch.Tensor] = None,
                   order: Optional[torch.Tensor] = None):
    """Split-KV partial attention.  Returns ``(partial_o, partial_lse, num_splits)``.
    q_scale and kv_scale are host numbers, or both 1-element fp32 device tensors (e.g. from
    quantize_fp8_sat_dynamic), which selects mla_decode_splitkv_dev_scales.  q_lens (int32
    [B] on the GPU) gives each request its own number of query tokens (<= Sq; the first
    q_lens[b] slots of q8[b]), through mla_decode_splitkv_ex; ctx_after (int32 [B] on the GPU)
    counts each request's context positions after the ones this call reads (a context shard
    other than the last); order (int32 [B] on the GPU, a permutation) is the order in which
    requests' workgroups are dispatched, longest first for mixed lengths.

    q8 [B, Sq, H, 576] uint8; kv_pool8 [pages, page_size, 576] uint8; page_table
    [B, max_pages] int32; seq_lens [B] int32.  partial_o [B, S, Sq*H, 512] fp16 (in units of
    kv_scale) and partial_lse [B, S, Sq*H] fp32 are allocated when not given.
    """
    _dev_tensor(q8, torch.uint8, "q8")
    _dev_tensor(kv_pool8, torch.uint8, "kv_pool8")
    _dev_tensor(page_table, torch.int32, "page_table")
    _dev_tensor(seq_lens, torch.int32, "seq_lens")
    B, Sq, H, d = q8.shape
    if d != D_KV or kv_pool8.dim() != 3 or kv_pool8.shape[2] != D_KV:
        raise ValueError("q8 and kv_pool8 rows must be 576 wide")
    page_size = kv_pool8.shape[1]
    if num_splits == 0 or rows_per_group == 0:
        plan = splitkv_plan(B, Sq, H, max_seq_len)
        num_splits = num_splits or plan.num_splits
        rows_per_group = rows_per_group or plan.rows_per_group
    rows = Sq * H
    if partial_o is None:
        partial_o = torch.empty((B, num_splits, rows, D_V), dtype=torch.float16,
                                device=q8.device)
    if partial_lse is None:
        partial_lse = torch.empty((B, num_splits, rows), dtype=torch.float32, device=q8.device)
    _dev_tensor(partial_o, torch.float16, "partial_o")
    _dev_tensor(partial_lse, torch.float32, "partial_lse")
    cap = min(partial_o.numel() // D_V, partial_lse.numel())
    dq, dk = _dev_scale(q_scale, "q_scale"), _dev_scale(kv_scale, "kv_scale")
    if dq != dk:
        raise ValueError("q_scale and kv_scale must both be host numbers or both device tensors")
    if q_lens is not None or ctx_after is not None or order is not None:
        for t, name in ((q_lens, "q_lens"), (ctx_after, "ctx_after"), (order, "order")):
            if t is not None:
                _dev_tensor(t, torch.int32, name)
                if t.numel() != B:
                    raise ValueError(f"{name} must hold one count per request")
        _check(_lib.mla_decode_splitkv_ex(
            _ptr(q8), _ptr(kv_pool8), _ptr(page_table), _ptr(seq_lens), _ptr(q_lens),
            _ptr(ctx_after), _ptr(order), B, Sq, H,
            page_size, page_table.shape[1], max_seq_len, 1.0 if dq else float(q_scale),
            1.0 if dk else float(kv_scale), _ptr(q_scale) if dq else None,
            _ptr(kv_scale) if dk else None, float(softmax_scale), num_splits, rows_per_group,
            _ptr(partial_o), _ptr(partial_lse), cap, _stream(q8.device)),
            "mla_decode_splitkv_ex")
        return partial_o, partial_lse, num_splits
    if dq:
        _check(_lib.mla_decode_splitkv_dev_scales(
            _ptr(q8), _ptr(kv_pool8), _ptr(page_table), _ptr(seq_lens), B, Sq, H, page_size,
            page_table.shape[1], max_seq_len, _ptr(q_scale), _ptr(kv_scale),
            float(softmax_scale), num_splits, rows_per_group, _ptr(partial_o),
            _ptr(partial_lse), cap, _stream(q8.device)), "mla_decode_splitkv_dev_scales")
        return partial_o, partial_lse, num_splits
    _check(_lib.mla_decode_splitkv(
        _ptr(q8), _ptr(kv_pool8), _ptr(page_table), _ptr(seq_lens), B, Sq, H, page_size,
        page_table.shape[1], max_seq_len, float(q_scale), float(kv_scale),
        float(softmax_scale), num_splits, rows_per_group, _ptr(partial_o), _ptr(partial_lse),
        cap, _stream(q8.device)), "mla_decode_splitkv")
    return partial_o, partial_lse, num_splits


def splitkv_combine(partial_o: torch.Tensor, partial_lse: torch.Tensor, q_tokens: int,
                    heads: int, v_scale: float, out: Optional[torch.Tensor] = None,
                    out_lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """LSE merge -> (out [B, Sq, H, 512] bf16, lse [B, Sq, H] fp32 or None).  partial_o is
    fp16 in units of v_scale (the KV scale), as decode_splitkv writes it; v_scale may be a
    1-element fp32 device tensor (mla_splitkv_combine_dev_scale)."""
    _dev_tensor(partial_o, torch.float16, "partial_o")
    _dev_tensor(partial_lse, torch.float32, "partial_lse")
    B, S = partial_lse.shape[0], partial_lse.shape[1]
    if partial_lse.shape[2] != q_tokens * heads or partial_o.shape[:3] != partial_lse.shape:
        raise ValueError("partial shapes do not match [B, S, Sq*H(, 512)]")
    dev = partial_o.device
    if out is None:
        out = torch.empty((B, q_tokens, heads, D_V), dtype=torch.bfloat16, device=dev)
    if out_lse is None and want_lse:
        out_lse = torch.empty((B, q_tokens, heads), dtype=torch.float32, device=dev)
    _dev_tensor(out, torch.bfloat16, "out")
    if out_lse is not None:
        _dev_tensor(out_lse, torch.float32, "out_lse")
    if _dev_scale(v_scale, "v_scale"):
        _check(_lib.mla_splitkv_combine_dev_scale(_ptr(partial_o), _ptr(partial_lse), B, S,
                                                  q_tokens, heads, _ptr(v_scale), _ptr(out),
                                                  _ptr(out_lse), _stream(dev)),
               "mla_splitkv_combine_dev_scale")
        return out, out_lse
    _check(_lib.mla_splitkv_combine(_ptr(partial_o), _ptr(partial_lse), B, S, q_tokens, heads,
                                    float(v_scale), _ptr(out), _ptr(out_lse), _stream(dev)),
           "mla_splitkv_combine")
    return out, out_lse


def splitkv_combine_partial(partial_o: torch.Tensor, partial_lse: torch.Tensor, q_tokens: int,
                            heads: int, out_o: torch.Tensor, out_lse: torch.Tensor,
                            out_batch_stride_rows: int = 0) -> None:
    """Merge the S splits of each (b, row) into one partial in the decode's format (fp16 in
    units of the KV scale, natural-log lse), written at row b * out_batch_stride_rows + r of
    out_o / out_lse (flat row views; default stride Sq*H).  To fill slice g of a
    [B, G, Sq*H] buffer, pass views starting at slice g and stride G*Sq*H."""
    _dev_tensor(partial_o, torch.float16, "partial_o")
    _dev_tensor(partial_lse, torch.float32, "partial_lse")
    if not out_o.is_cuda or out_o.dtype != torch.float16 or not out_lse.is_cuda or \
            out_lse.dtype != torch.float32:
        raise ValueError("out_o must be fp16 and out_lse fp32 on the GPU")
    B, S = partial_lse.shape[0], partial_lse.shape[1]
    R = q_tokens * heads
    if partial_lse.shape[2] != R or partial_o.shape[:3] != partial_lse.shape:
        raise ValueError("partial shapes do not match [B, S, Sq*H(, 512)]")
    stride = out_batch_stride_rows or R
    # the rows written lie within the views given
    last = (B - 1) * stride + R
    if out_lse.untyped_storage().nbytes() < (out_lse.storage_offset() + last) * 4 or \
            out_o.untyped_storage().nbytes() < (out_o.storage_offset() + last * D_V) * 2:
        raise ValueError("out_o / out_lse are too small for the rows written")
    _check(_lib.mla_splitkv_combine_partial(_ptr(partial_o), _ptr(partial_lse), B, S, q_tokens,
                                            heads, _ptr(out_o), _ptr(out_lse), int(stride),
                                            _stream(partial_o.device)),
           "mla_splitkv_combine_partial")


def decode_noalloc(q8: torch.Tensor, kv_pool8: torch.Tensor, page_table: torch.Tensor,
                   seq_lens: torch.Tensor, q_scale: float, kv_scale: float, softmax_scale: float,
                   max_seq_len: int, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                   out_lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Decode + combine through mla_decode_noalloc (the split partials stay in the library's
    own device array; the C call allocates nothing).  Returns ``(out bf16 [B, Sq, H, 512],
    lse fp32 [B, Sq, H] or None)``; outputs not given are allocated here with torch."""
    _dev_tensor(q8, torch.uint8, "q8")
    _dev_tensor(kv_pool8, torch.uint8, "kv_pool8")
    _dev_tensor(page_table, torch.int32, "page_table")
    _dev_tensor(seq_lens, torch.int32, "seq_lens")
    B, Sq, H, d = q8.shape
    if d != D_KV or kv_pool8.dim() != 3 or kv_pool8.shape[2] != D_KV:
        raise ValueError("q8 and kv_pool8 rows must be 576 wide")
    dev = q8.device
    if out is None:
        out = torch.empty((B, Sq, H, D_V), dtype=torch.bfloat16, device=dev)
    if out_lse is None and want_lse:
        out_lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    _dev_tensor(out, torch.bfloat16, "out")
    if out.numel() != B * Sq * H * D_V:
        raise ValueError("out must be [B, Sq, H, 512]")
    if out_lse is not None:
        _dev_tensor(out_lse, torch.float32, "out_lse")
        if out_lse.numel() != B * Sq * H:
            raise ValueError("out_lse must be [B, Sq, H]")
    _check(_lib.mla_decode_noalloc(
        _ptr(q8), _ptr(kv_pool8), _ptr(page_table), _ptr(seq_lens), B, Sq, H,
        kv_pool8.shape[1], page_table.shape[1], int(max_seq_len), float(q_scale),
        float(kv_scale), float(softmax_scale), int(num_splits), _ptr(out), _ptr(out_lse),
        _stream(dev)), "mla_decode_noalloc")
    return out, out_lse


def hbm_read_probe(buf: torch.Tensor, out: torch.Tensor, grid: int) -> None:
    """Diagnostics: stream every byte of buf (a multiple of 32 KiB) from HBM; one uint32
    XOR-fold per workgroup into out[:grid].  Used to measure the read rate in benchmarks."""
    if not buf.is_cuda or not out.is_cuda or out.dtype != torch.int32 or out.numel() < grid:
        raise ValueError("buf and out must be device tensors, out int32 with >= grid elements")
    _check(_lib.mla_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                   int(grid), _stream(buf.device)), "mla_hbm_read_probe")


def decode(q8, kv_pool8, page_table, seq_lens, q_scale, kv_scale, softmax_scale, max_seq_len,
           num_splits: int = 0, rows_per_group: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Partial attention followed by the combine: (out bf16, lse fp32)."""
    po, pl, _ = decode_splitkv(q8, kv_pool8, page_table, seq_lens, q_scale, kv_scale,
                               softmax_scale, max_seq_len, num_splits, rows_per_group)
    return splitkv_combine(po, pl, q8.shape[1], q8.shape[2], kv_scale)
