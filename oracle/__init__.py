"""CPU oracle for the fused MXFP8 QKV projection, across-heads QK RMSNorm and rotate-half RoPE.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 NumPy statement of what the
method computes, written from the source pages:

  [QKV-CTE]   "Kernel reference: qkv_cte -- Wan2.2 additions to the NKI Library QKV CTE MXFP8
              projection" (sections "Applies to", "Upstream behavior", "Design 1)" .. "Design 5)",
              "Interface").
  [RMSNORM-MX] "RMSNorm MX Prefill Kernel API Reference" (parameters ``eps``, ``residual``,
              ``unpadded_hidden_size``, ``qmx_output_dtype``, ``emit_norm_bf16``).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import it.  It
shares no code with the HIP library (``rope_mxfp8_qkv_amd``) and never imports it; the only
module both sides use is ``synth`` (seeded random inputs, no arithmetic of the method).

Every function here is pinned by CPU tests against something other than itself (library
codecs, exact rational brute force, closed forms, invariants); see ``tests/test_oracle_*.py``.
"""
from .codecs import (e4m3_decode, e4m3_encode, e8m0_decode, bf16_round_f32, bf16_to_f64,
                     f64_to_bf16)
from .rowmx import rowmx_quantize, rowmx_unpack
from .mxweight import mx_weight_quantize, mx_weight_decode
from .gemm import project, segment_ssq, abs_term_sum
from .norm_rope import inv_rms, norm_rope
from .producer import rmsnorm_rowmx, rmsnorm_mx
from .mxact import mx_block_quantize, mx_block_decode
from .layouts import bsd_to_nbsd, nbsd_to_bsd
from .headnorm import head_norm_rope, RMS_NORM, LAYER_NORM

__all__ = [
    "e4m3_decode", "e4m3_encode", "e8m0_decode", "bf16_round_f32", "bf16_to_f64", "f64_to_bf16",
    "rowmx_quantize", "rowmx_unpack", "mx_weight_quantize", "mx_weight_decode",
    "project", "segment_ssq", "abs_term_sum", "inv_rms", "norm_rope", "rmsnorm_rowmx", "rmsnorm_mx", "mx_block_quantize", "mx_block_decode", "bsd_to_nbsd", "nbsd_to_bsd",
    "head_norm_rope", "RMS_NORM", "LAYER_NORM",
]
