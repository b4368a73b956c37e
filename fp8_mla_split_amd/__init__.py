"""FP8 MLA split-KV decode for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmla.so`` (hand-written HIP kernels, declared in
``include/mla.h``); this package only marshals arguments to it.  The binding is loaded on
first use of any public name, and that fails loudly if the library has not been built
(``python -m fp8_mla_split_amd.build``).  The build module itself imports without it.
"""
_PUBLIC = (
    "MLAError", "Plan", "QUANTIZE_DYNAMIC_WORKSPACE_BYTES", "decode", "decode_noalloc",
    "decode_splitkv",
    "hbm_read_probe", "kv_append_fp8_sat", "kv_append_rope_fp8_sat",
    "lib_path", "quantize_fp8_sat", "quantize_fp8_sat_dynamic", "splitkv_combine",
    "splitkv_combine_partial",
    "splitkv_plan", "status_string",
)
__all__ = list(_PUBLIC)


def __getattr__(name):
    if name in _PUBLIC:
        from . import mla as _mla
        return getattr(_mla, name)
    raise AttributeError(name)
