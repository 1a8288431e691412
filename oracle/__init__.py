"""CPU oracle for the small-batch decode MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It is a plain, slow, FP64 numpy implementation written from the pages' description
of the layer, sharing no code, table or constant generator with the HIP kernels.

Modules:
  formats -- E2M1 / E4M3 / E8M0 / BF16 decode tables and nearest-even encoders
  quant   -- Four-Over-Six NVFP4 and FP8 per-token quantizers (exact FP32 emulation),
             weight dequantization
  router  -- FP64 router logits, sigmoid top-k, renormalised combine weights
  layer   -- expert MLPs (SwiGLU), activation re-quantization, weighted combine
  norm    -- RMSNorm of the residual stream before the layer, residual add after it

Every function is pinned by tests under tests/ (hand-worked tables, brute force on
small inputs, closed forms, exact rational arithmetic). The full-layer composition
has no printed worked example on the pages: it is pinned only through its parts and
the closed-form layers in tests/test_oracle_layer.py.
"""
from . import formats, quant, router, layer, norm  # noqa: F401
