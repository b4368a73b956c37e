"""FP8 MLA split-KV decode for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmla.so`` (hand-written HIP kernels, declared in
``include/mla.h``); this package only marshals arguments to it.  Importing fails loudly if
the library has not been built (``python -m fp8_mla_split_amd.build``).
"""
from .mla import (  # noqa: F401
    MLAError,
    Plan,
    decode,
    decode_splitkv,
    lib_path,
    quantize_fp8_sat,
    splitkv_combine,
    splitkv_plan,
    status_string,
)
