"""CPU oracle for the block-scaled FP8 (E4M3) W8A8 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, header, table
or helper with the HIP library under ``block_scaled_fp8_quant_amd/``; the
two meet only in the seeded input generators of ``synth/``.

What it computes (sources are web pages about NVIDIA NeMo RL's FP8 recipe):

* "NVIDIA NeMo RL достигает ускорения на 48% благодаря сквозному обучению с
  точностью FP8" (greentreeone.com, news 1041474), section «Технический
  прорыв»: block-quantized FP8 in the E4M3 format, one scale per 128x128
  weight block and per 1x128 activation group; linear layers run their math
  in FP8.
* The upppp.jp NeMo RL FP8 article (upppp.jp/?p=471), section «設定方法», and
  the greentreeone.com article, section «Почему это важно для экономики ИИ»:
  an option restricts scale factors to powers of two.
* Both pages (upppp.jp «まとめ», greentreeone.com «Реальные прирост
  производительности»): the recipe also holds on a mixture-of-experts model,
  which is served here by a grouped GEMM over expert-sorted rows.
* Both pages (upppp.jp «重要度サンプリングで精度を保つ», greentreeone.com
  «Реальные прирост производительности»): the quantization kernels are
  overhead and their fusion is the way past it; ``producers`` holds the two
  producers fused with the activation quantization (RMSNorm, SiLU * up).
* Both pages (upppp.jp «KVキャッシュとAttentionにも拡張», greentreeone.com
  «Реальные прирост производительности»): the KV cache in FP8, with the
  Q/K/V scales recalibrated after every training step; ``kv_cache`` holds the
  per-tensor recalibration and the quantize-and-write of K and V.
* FP8 training (upppp.jp «FP8適用の難所：数値のズレ問題», greentreeone.com
  «Технический прорыв»): ``backward`` holds the dgrad and wgrad GEMMs under
  the same quantization rule along each GEMM's contraction dimension.
* Both pages (upppp.jp «KVキャッシュとAttentionにも拡張», greentreeone.com
  «Реальные прирост производительности»): attention in FP8 over the FP8 KV
  cache; ``attention`` holds the decode step's attention over the paged cache
  and the prefill step's (a prompt's new tokens, causally).

The pages give no scale formula, no E4M3 variant, no rounding mode and no
accumulation scheme. The readings taken where they are silent are written
next to each function: OCP E4M3 ("FN": max 448, no infinities), scale =
amax/448 in fp32 (or the smallest power of two >= amax/448), quotient x/s
rounded once to fp32 by IEEE division, then round-to-nearest-even into E4M3
with saturation at +-448, fp32 scales stored as dequantisation multipliers,
Y = X W^T accumulated exactly (fp64) and compared with tolerance.

Everything is plain numpy in float64 (every value handled is exactly
representable there), with Python ``fractions`` for the brute-force pins in
the tests. Each function states what pins it; no function is unpinned.
"""

from .e4m3 import (
    E4M3_MAX,
    decode_table,
    decode,
    encode,
    encode_bruteforce,
)
from .quant import (
    GROUP,
    bf16_values,
    group_scale,
    quantize_values,
    quant_act_ref,
    quant_weight_ref,
)
from .producers import (
    rmsnorm_ref,
    silu_mul_ref,
    round_bf16,
)
from .kv_cache import (
    qkv_amax_ref,
    kv_scales_ref,
    kv_quantize_ref,
    kv_cache_write_ref,
)
from .backward import (
    quant_act_t_ref,
    quant_weight_t_ref,
    gemm_rowscaled_ref,
    dgrad_ref,
    wgrad_ref,
    padded_offsets,
    quant_act_t_grouped_ref,
    grouped_dgrad_ref,
    grouped_wgrad_ref,
)
from .attention import decode_attention_ref, prefill_attention_ref
from .gemm import (
    dequant_act,
    dequant_weight,
    gemm_ref,
    gemm_ref_blas,
    grouped_gemm_ref,
    gemm_rows_ref,
    tolerance_ok,
)

__all__ = [
    "E4M3_MAX", "decode_table", "decode", "encode", "encode_bruteforce",
    "GROUP", "bf16_values", "group_scale", "quantize_values",
    "quant_act_ref", "quant_weight_ref",
    "dequant_act", "dequant_weight", "gemm_ref", "gemm_ref_blas",
    "grouped_gemm_ref", "gemm_rows_ref", "tolerance_ok",
    "rmsnorm_ref", "silu_mul_ref", "round_bf16",
    "qkv_amax_ref", "kv_scales_ref", "kv_quantize_ref", "kv_cache_write_ref",
    "quant_act_t_ref", "quant_weight_t_ref", "gemm_rowscaled_ref", "dgrad_ref", "wgrad_ref",
    "padded_offsets", "quant_act_t_grouped_ref", "grouped_dgrad_ref", "grouped_wgrad_ref",
    "decode_attention_ref",
    "prefill_attention_ref",
]
