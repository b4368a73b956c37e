"""CPU oracle for FP8 MLA split-KV decode -- TEST INFRASTRUCTURE ONLY.

Plain, slow NumPy float64 code that states what the decode path computes.  It
shares nothing with the GPU path (no kernels, headers, tables, constants or
helpers); the only code both sides use is the seeded input generator in
``synthetic/``, which holds none of the method's arithmetic.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product library never does.

Sources cited in this package:

* [A]  the arex-research.com page "SGLang 与 Miles 团队称在预发布 Vera Rubin 上跑通
  Kimi K3 推理和端到端 RL，自测 FP8 MLA 提速最高约 20%".  [A/MLA] is its section
  "Kimi K3 的 MLA：更深的流水线、更快的 split-KV 归约", whose list has four items:
  (1) deeper MLA pipeline, (2) faster split-KV reduction, (3) 64-way split-KV,
  (4) native (saturating) FP8 conversion.
* [B]  the ai.newsbites.today page "LMSYS、NVIDIA Rubin向けの高速化成果を発表",
  section "MLAアテンションのパイプライン深化" and table "世代間スペック比較と最適化による効果".
* [OCP] the OCP 8-bit floating point specification (OFP8), E4M3 encoding.  The
  pages only give the +-448 bound, which singles out the E4M3 variant that has
  no infinities (max normal 448, NaN = S.1111.111).

Pinning (what each function is checked against, in ``tests/test_oracle_*``):

* ``e4m3_table``         OCP spot values and ``torch.float8_e4m3fn`` for all 256 codes.
* ``quantize_e4m3_sat``  ``clamp(+-448)`` followed by torch's RNE fp8 cast on a
                         structured sweep of fp32 patterns; hand-worked ties;
                         the saturation rule of [A/MLA] item (4).
* ``attention_fp64``     closed forms on tiny inputs; float64
                         ``scaled_dot_product_attention`` with an explicit
                         causal mask; paged == contiguous; head independence.
                         Per-request query counts (``q_lens``): a hand-written
                         loop over a 2-of-4-token request, empty requests, and
                         equality with a call holding only those slots.
* ``split_partials_fp64`` / ``combine_fp64``  S = 1 identity, the two-split
                         closed form, and split-count independence.
* ``bf16_bits_to_f32``   torch's bfloat16 -> float32 conversion on all 65536
                         patterns, and spot values.
* ``dynamic_quantize``   the scale maps the tensor's largest magnitude to the code
                         0x7E exactly; bf16 and fp32 sources of the same values agree.
* ``append_kv_fp8``      appending a request's rows one step at a time and reading
                         them back through the attention's own gather gives the
                         quantised rows in order; bytes outside the new rows never
                         change; one T-row append equals T one-row appends.

* ``rope_rotate_f32`` / ``append_kv_rope_fp8``  the fp64 rotation of the same fp32 inputs
                         (within the bound of three fp32 roundings); angle 0 is the plain
                         append and a quarter turn maps (x0, x1) to (-x1, x0) exactly; a
                         standard RoPE table agrees with torch's complex multiplication;
                         latent columns and positions past the table are untouched.

No function here is "parity unpinned".
"""
from .e4m3 import (  # noqa: F401
    E4M3_MAX,
    decode_e4m3,
    e4m3_table,
    per_tensor_scale,
    quantize_e4m3_sat,
)
from .cache import (  # noqa: F401
    append_kv_fp8,
    append_kv_rope_fp8,
    bf16_bits_to_f32,
    dynamic_quantize,
    rope_rotate_f32,
)
from .attention import (  # noqa: F401
    attention_fp64,
    combine_fp64,
    even_partition,
    gather_kv_rows,
    split_partials_fp64,
)
