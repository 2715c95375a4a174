"""CPU oracle for the NVFP4 W4A4 hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path (the C-ABI
library and its Python binding) never does, and it shares no code, table or
constant generator with that path.

Sources (the pages this follows):
  [P1] "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
       Recurrent Half of a Hybrid 27B LLM" -- arxiv-wiki summary page,
       sections "접근 방법" (approach) and "개발자 관점" (developer view).
  [P2] the same paper's listing page (shd-paper), English abstract.
  [P3] "論文解説: Gated DeltaNet はなぜ4bit量子化に耐えるのか" -- explainer
       page, sections "前提1" (what rounding to 4 bits means) and "前提2"
       (what Gated DeltaNet computes).

Two tiers:
  * exact  -- pure Python on fractions.Fraction and int; tiny inputs only.
  * fast   -- vectorised numpy float64 whose every rounding decision is
              provably the exact one (argument in quantize.py); full sizes.
The exact tier pins the fast tier (tests/test_oracle_pins.py).

Every function is pinned by a test against something other than itself
(closed forms, library routines, brute force); none is "parity unpinned".
"""
from .formats import (E2M1_MAG, e2m1_decode, e4m3_decode, e4m3_decode_table,
                      e2m1_rne_sat_exact, e4m3_rne_sat_exact, fp32_rne_exact,
                      bf16_rne_from_f64, GLOBAL_DIVISOR)
from .quantize import (quantize, quantize_exact, dequantize, global_scale,
                       block_scales, encode_elements,
                       unpack_codes, pack_codes, dequantize_f32,
                       dequantize_bf16, error_stats)
from .harmonize import harmonize, harmonize_exact
from .fp8kv import (kv_amax, kv_scale, kv_cast, kv_decode, kv_cast_exact,
                    kv_scale_exact)
from .gemm import (gemm_exact_int, gemm_f64, gemm_f64_rows_cols,
                   gemm_f64_row_blocks, gate_alpha, gate_beta, decoded_units,
                   gdn_gates)

__all__ = [
    "E2M1_MAG", "e2m1_decode", "e4m3_decode", "e4m3_decode_table",
    "e2m1_rne_sat_exact", "e4m3_rne_sat_exact", "fp32_rne_exact",
    "bf16_rne_from_f64", "GLOBAL_DIVISOR",
    "quantize", "quantize_exact", "dequantize", "global_scale",
    "unpack_codes", "pack_codes", "block_scales", "encode_elements",
    "dequantize_f32", "dequantize_bf16", "error_stats",
    "harmonize", "harmonize_exact",
    "kv_amax", "kv_scale", "kv_cast", "kv_decode", "kv_cast_exact",
    "kv_scale_exact",
    "gemm_exact_int", "gemm_f64", "gemm_f64_rows_cols", "gemm_f64_row_blocks",
    "gate_alpha",
    "gate_beta", "decoded_units", "gdn_gates",
]
