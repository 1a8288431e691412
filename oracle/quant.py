"""Activation quantizers and weight dequantization (CPU oracle).

Test infrastructure (see oracle/__init__.py).

* quantize_nvfp4_4o6 -- "Inkling 2 Small on vLLM: Day-0 Support", section on
  mixed-precision MoE and Four-Over-Six NVFP4: NVFP4 activations carry a per-token
  global scale and, per 16-element block, the quantizer tries scaling the block
  maximum to 6 and to 4 and keeps the candidate with the lower reconstruction error
  (MAE). The per-token global scale is amax / (6 * 448).
* quantize_fp8_token -- "Day 0 support for Mistral Large 4 on vLLM", AMD section,
  MXFP4 experts: a8w4 runs MXFP4 experts on FP8 activations with dynamic scales;
  here one FP32 scale per row, amax / 448.
* quantize_mxfp4 -- the same page, ROCm implementation details (load-time expert
  requantization): each expert is dequantized to BF16 and requantized to MXFP4, E2M1
  values with one E8M0 scale per 32. The scale follows the OCP MX v1.0 rule: shared
  exponent floor(log2(block amax)) minus 2 (the largest E2M1 exponent), clamped to the
  E8M0 range [-127, 127]; elements are the block values times 2^-exponent, rounded to
  E2M1 (nearest, ties to even, saturating at 6). An all-zero block takes the smallest
  scale, 2^-127 (byte 0), and zero codes carrying the input signs.
* quantize_mxfp8 -- the same OCP rule for MXFP8 (the Inkling page's MXFP8 expert layers):
  shared exponent floor(log2(block amax)) minus 8 (the largest E4M3 exponent), clamped to
  [-127, 127]; elements rounded to E4M3 (nearest, ties to even, saturating at 448).
* dequant_fp8_block -- the same page's load path starts from a block-scaled FP8
  checkpoint: E4M3 expert weights with their block scales, each expert dequantized to
  BF16 before the MXFP4 requantization. Readings: one FP32 scale per block_rows x
  block_cols block of a [rows, cols] matrix (scales [ceil(rows/br), ceil(cols/bc)], the
  edge blocks ragged); a value is E4M3(code) times its block's scale, one FP32 product
  (rounded to nearest even), then rounded to BF16 (nearest even). NaN codes are outside
  the domain.
* quantize_nvfp4_weights -- BF16 -> NVFP4 weight requantization (the load path's other
  target format; the pages do not spell its rule out): the two-level NVFP4 recipe, one
  FP32 scale per tensor g = amax / 2688 and, per 16-block, the Four-Over-Six arithmetic
  above with the target 6 only (no 4 candidate).

The pages fix neither the floating-point operation order nor the zero and saturation
cases. The quantizer is defined as exact IEEE FP32 operations in the order written
below (numpy float32 arithmetic is correctly rounded and never fused), so a GPU
implementation can reproduce its codes and scales bit for bit.
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_TABLE, E4M3_TABLE, E8M0_TABLE, bf16_to_f64, e2m1_encode,
                      e4m3_encode_satfinite, pack_fp4, unpack_fp4)
from .norm import to_bf16_bits

F32 = np.float32
NVFP4_BLOCK = 16
MX_BLOCK = 32
E4M3_MAX = F32(448.0)
NVFP4_GLOBAL_DIV = F32(6.0 * 448.0)  # 2688: the largest E2M1 value times the largest E4M3 value


def tree_sum16(e: np.ndarray) -> np.ndarray:
    """FP32 sum over the last axis (length 16) in a fixed pairwise tree.

    Level 1 adds element i and i+8, level 2 adds i and i+4 of the result, then i and
    i+2, then the last pair. A 64-wide xor-shuffle reduction by 8, 4, 2, 1 over 16
    lanes performs the same additions.
    """
    e = np.asarray(e, dtype=F32)
    assert e.shape[-1] == 16
    s = e[..., :8] + e[..., 8:]
    s = s[..., :4] + s[..., 4:]
    s = s[..., :2] + s[..., 2:]
    return s[..., 0] + s[..., 1]


def _candidate(xb: np.ndarray, m: np.ndarray, g: np.ndarray, c: F32):
    """One Four-Over-Six candidate for blocks xb [..., 16] (FP32), block max m, row scale g.

    Returns (scale byte, codes [..., 16], FP32 error sum).
    """
    u = (m / g) / c                                   # two FP32 divisions, in this order
    sbyte = e4m3_encode_satfinite(u)
    S = E4M3_TABLE[sbyte].astype(F32)                 # exact: E4M3 values fit in FP32
    d = (S * g).astype(F32)                           # element scale, FP32 product
    zero = d == 0                                     # scale underflowed (S = 0 or S*g tiny)
    d_safe = np.where(zero, F32(1.0), d)
    q = e2m1_encode(xb / d_safe[..., None])
    r = (E2M1_TABLE[q].astype(F32) * d_safe[..., None]).astype(F32)
    err_el = np.abs(xb - r).astype(F32)
    # A zero element scale reconstructs every element as zero: codes keep only the sign.
    q = np.where(zero[..., None], (np.signbit(xb).astype(np.uint8) << 3), q).astype(np.uint8)
    err_el = np.where(zero[..., None], np.abs(xb), err_el).astype(F32)
    return sbyte, q, tree_sum16(err_el)


def quantize_nvfp4_4o6(x: np.ndarray):
    """Four-Over-Six NVFP4 quantization of each row of ``x`` ([rows, n], n % 16 == 0).

    Per row, in FP32:
      1. a = max |x_i| over the row.
      2. a == 0: g = 0, all scale bytes 0, every code keeps only x_i's sign bit.
      3. g = a / 2688.
      4. Per 16-block with maximum m, for c in (6, 4):
           u_c = (m / g) / c,  S_c = E4M3(u_c) (nearest-even, saturating at 448),
           d_c = S_c * g,      q_i = E2M1(x_i / d_c) (nearest-even, saturating at 6),
           err_c = tree-sum over the block of |x_i - v(q_i) * d_c|.
         d_c == 0 encodes the block as zeros (sign bits kept) with err_c = sum |x_i|.
      5. Keep c = 4 only if err_4 < err_6 (ties go to 6).
    Returns codes [rows, n/2] (element 2i in the low nibble), scale bytes [rows, n/16],
    g [rows] (FP32) and the choice [rows, n/16] in {4, 6}.
    """
    x = np.asarray(x, dtype=F32)
    rows, n = x.shape
    assert n % NVFP4_BLOCK == 0, "row length must be a multiple of 16"
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_nvfp4_4o6: non-finite input")
    nb = n // NVFP4_BLOCK
    xb = x.reshape(rows, nb, NVFP4_BLOCK)
    a = np.max(np.abs(x), axis=1) if n else np.zeros(rows, F32)
    a = a.astype(F32)
    live = a > 0
    g = np.where(live, a / NVFP4_GLOBAL_DIV, F32(0.0)).astype(F32)
    g_safe = np.where(live, g, F32(1.0))[:, None]     # dead rows are overwritten below
    m = np.max(np.abs(xb), axis=2).astype(F32)
    s6, q6, e6 = _candidate(xb, m, g_safe, F32(6.0))
    s4, q4, e4 = _candidate(xb, m, g_safe, F32(4.0))
    pick4 = e4 < e6
    sbytes = np.where(pick4, s4, s6).astype(np.uint8)
    codes = np.where(pick4[..., None], q4, q6).astype(np.uint8)
    choice = np.where(pick4, 4, 6).astype(np.uint8)
    dead = ~live
    sbytes[dead] = 0
    codes[dead] = (np.signbit(xb[dead]).astype(np.uint8) << 3)
    choice[dead] = 6
    return pack_fp4(codes.reshape(rows, n)), sbytes, g, choice


def dequant_nvfp4_rows(codes: np.ndarray, sbytes: np.ndarray, g) -> np.ndarray:
    """NVFP4 rows -> float64: v(q_i) * S(block) * g, computed in FP64.

    ``g`` is a scalar (one per tensor) or one value per row.
    """
    q = unpack_fp4(codes)
    S = np.repeat(E4M3_TABLE[sbytes], NVFP4_BLOCK, axis=-1)
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 1:
        g = g[:, None]
    return E2M1_TABLE[q] * S * g


def quantize_fp8_token(x: np.ndarray):
    """FP8-E4M3 quantization with one FP32 scale per row ([rows, n]).

    a = max |x_i|; a == 0 gives s = 0 and codes that keep only the sign; otherwise
    s = a / 448 and q_i = E4M3(x_i / s) (nearest-even, saturating at 448).
    Returns codes [rows, n] (bytes) and s [rows] (FP32).
    """
    x = np.asarray(x, dtype=F32)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_fp8_token: non-finite input")
    a = (np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], F32)).astype(F32)
    live = a > 0
    s = np.where(live, a / E4M3_MAX, F32(0.0)).astype(F32)
    s_safe = np.where(live, s, F32(1.0))[:, None]
    codes = e4m3_encode_satfinite((x / s_safe).astype(F32))
    codes[~live] = (np.signbit(x[~live]).astype(np.uint8) << 7)
    return codes, s


def dequant_fp8_token(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[codes] * np.asarray(s, dtype=np.float64)[:, None]


def quantize_mxfp4(x: np.ndarray):
    """MXFP4 of rows x [rows, cols] (FP32 values, cols % 32 == 0): returns (packed codes
    [rows, cols/2] uint8, element 2i in the low nibble; E8M0 scale bytes [rows, cols/32])."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    xb = x.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(axis=2).astype(np.float64)
    _, e = np.frexp(amax)                          # amax = m * 2^e, m in [0.5, 1): floor(log2) = e - 1
    shared = np.where(amax > 0, e - 1 - 2, -127)
    shared = np.clip(shared, -127, 127).astype(np.int64)
    y = np.ldexp(xb.astype(np.float64), -shared[:, :, None]).astype(np.float32)   # exact scaling
    codes = e2m1_encode(y).reshape(rows, cols)
    return pack_fp4(codes), (shared + 127).astype(np.uint8)


def quantize_mxfp8(x: np.ndarray):
    """MXFP8 (E4M3) of rows x [rows, cols] (FP32 values, cols % 32 == 0): returns (codes
    [rows, cols] uint8, E8M0 scale bytes [rows, cols/32])."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    xb = x.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(axis=2).astype(np.float64)
    _, e = np.frexp(amax)                          # floor(log2(amax)) = e - 1
    shared = np.where(amax > 0, e - 1 - 8, -127)
    shared = np.clip(shared, -127, 127).astype(np.int64)
    y = np.ldexp(xb.astype(np.float64), -shared[:, :, None]).astype(np.float32)   # exact scaling
    return e4m3_encode_satfinite(y).reshape(rows, cols), (shared + 127).astype(np.uint8)


def dequant_fp8_block(codes: np.ndarray, scales: np.ndarray, block_rows: int, block_cols: int) -> np.ndarray:
    """Block-scaled FP8 weights to BF16 bit patterns: codes [rows, cols] E4M3 bytes, scales
    [ceil(rows/block_rows), ceil(cols/block_cols)] FP32. Element (r, c) takes the scale of
    block (r // block_rows, c // block_cols); its value is the FP32 product E4M3(code) *
    scale (E4M3 values are exact in FP32; numpy's float32 product is correctly rounded),
    then rounded once more, to BF16 with ties to even. Returns uint16 [rows, cols]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    s = np.asarray(scales, dtype=np.float32)
    if s.shape != (-(-rows // block_rows), -(-cols // block_cols)):
        raise ValueError("scales must be [ceil(rows / block_rows), ceil(cols / block_cols)]")
    vals = E4M3_TABLE[codes]
    if not np.all(np.isfinite(vals)):
        raise ValueError("dequant_fp8_block: NaN codes")
    per = s[(np.arange(rows) // block_rows)[:, None], (np.arange(cols) // block_cols)[None, :]]
    prod = vals.astype(np.float32) * per                       # one FP32 rounding
    if not np.all(np.isfinite(prod)):
        raise ValueError("dequant_fp8_block: product outside FP32")
    return to_bf16_bits(prod.astype(np.float64))              # then BF16


def requant_fp8_block_mxfp4(codes: np.ndarray, scales: np.ndarray, block_rows: int, block_cols: int):
    """The load path from a block-scaled FP8 checkpoint: dequant_fp8_block, then
    quantize_mxfp4 of those BF16 values. Returns (packed E2M1 codes, E8M0 scale bytes)."""
    bits = dequant_fp8_block(codes, scales, block_rows, block_cols)
    return quantize_mxfp4(bf16_to_f64(bits).astype(np.float32))


def quantize_nvfp4_weights(x: np.ndarray):
    """NVFP4 of tensors x [n, rows, cols] (FP32 values, cols % 16 == 0), one global scale
    per tensor: returns (packed codes [n, rows, cols/2], scale bytes [n, rows, cols/16],
    g [n] FP32). Per tensor, in FP32: a = max |x|; a == 0 gives g = 0, scale bytes 0 and
    sign-only codes; else g = a / 2688 and every 16-block takes the c = 6 candidate."""
    x = np.asarray(x, dtype=F32)
    n, rows, cols = x.shape
    if cols % NVFP4_BLOCK:
        raise ValueError("cols must be a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_nvfp4_weights: non-finite input")
    xb = x.reshape(n, rows * cols // NVFP4_BLOCK, NVFP4_BLOCK)
    a = np.abs(x).reshape(n, -1).max(axis=1).astype(F32)
    live = a > 0
    g = np.where(live, a / NVFP4_GLOBAL_DIV, F32(0.0)).astype(F32)
    g_safe = np.where(live, g, F32(1.0))[:, None]
    m = np.max(np.abs(xb), axis=2).astype(F32)
    sbytes, q, _ = _candidate(xb, m, g_safe, F32(6.0))
    sbytes = np.where(live[:, None], sbytes, 0).astype(np.uint8)
    q = np.where(live[:, None, None], q, (np.signbit(xb).astype(np.uint8) << 3)).astype(np.uint8)
    return (pack_fp4(q.reshape(n * rows, cols)).reshape(n, rows, cols // 2),
            sbytes.reshape(n, rows, cols // NVFP4_BLOCK), g)


def dequant_weights(fmt: str, codes: np.ndarray, scales, gscale) -> np.ndarray:
    """One weight tensor [rows][K] in storage format ``fmt`` -> float64 [rows][K].

    NVFP4: v(E2M1) * S(E4M3 per 16 along K) * g (FP32 per tensor).
    MXFP4: v(E2M1) * 2^(E8M0 per 32 along K - 127).
    MXFP8: v(E4M3) * 2^(E8M0 per 32 along K - 127).
    BF16: the value itself.
    All products are formed in FP64 and are exact.
    """
    if fmt == "bf16":
        return bf16_to_f64(codes)
    if fmt == "nvfp4":
        return dequant_nvfp4_rows(codes, scales, float(gscale))
    if fmt == "mxfp4":
        return E2M1_TABLE[unpack_fp4(codes)] * np.repeat(E8M0_TABLE[scales], MX_BLOCK, axis=-1)
    if fmt == "mxfp8":
        return E4M3_TABLE[codes] * np.repeat(E8M0_TABLE[scales], MX_BLOCK, axis=-1)
    raise ValueError(fmt)
