"""Element and scale formats: decode tables and round-to-nearest-even encoders.

Test infrastructure (see oracle/__init__.py): plain numpy, written from the format
definitions, sharing nothing with the GPU path.

The pages name the formats without defining their bits: NVFP4 (E2M1 values with an
E4M3 scale per 16 elements and an FP32 global scale) in "Inkling 2 Small on vLLM:
Day-0 Support", section on mixed-precision MoE and Four-Over-Six NVFP4; OCP MXFP4
(E2M1 values with one E8M0 scale per 32 values) and MXFP8 in "Day 0 support for
Mistral Large 4 on vLLM", ROCm implementation details, MXFP4 experts at load. The
bit layouts below are the OCP Microscaling v1.0 definitions of E2M1, E4M3 and E8M0.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes for the 3-bit code eem (exponent bias 1, one mantissa bit).
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code s|ee|m. No infinities or NaNs; code 8 is -0."""
    mag = E2M1_MAGNITUDES[code & 7]
    return -mag if code & 8 else mag


def e4m3_value(byte: int) -> float:
    """Value of an OCP E4M3 byte s|eeee|mmm, exponent bias 7.

    Exponent field 0 is subnormal (m * 2^-9); 0x7F and 0xFF are NaN; the largest
    finite magnitude is 448 (0x7E). There are no infinities.
    """
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e8m0_value(byte: int) -> float:
    """Value of an E8M0 scale byte: 2^(byte - 127); 0xFF is NaN. No sign, no zero."""
    if byte == 0xFF:
        return float("nan")
    return 2.0 ** (int(byte) - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64. BF16 is the top half of an FP32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _round_to_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value to each non-negative ``mag``.

    ``grid`` is increasing and indexed by code, so the least significant code bit is
    the mantissa's last bit. A value exactly halfway between two grid points takes
    the even code. Values above the last point take the last point (saturation).
    Comparisons are against exact midpoints, so no distance is ever rounded.
    """
    mag = np.asarray(mag, dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2.0          # exact: grid values have short mantissas
    idx = np.searchsorted(mids, mag, side="left")  # number of midpoints strictly below
    tie = np.zeros(mag.shape, dtype=bool)
    inside = idx < len(mids)
    tie[inside] = mids[idx[inside]] == mag[inside]
    # On a tie idx is the lower neighbour; keep it if its code is even, else go up.
    up = tie & (idx % 2 == 1)
    return (idx + up).astype(np.int64)


_E2M1_GRID = np.array(E2M1_MAGNITUDES, dtype=np.float64)
_E4M3_GRID = E4M3_TABLE[:0x7F]                 # 0x00 .. 0x7E: 0, subnormals, normals to 448


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """FP32 values -> E2M1 codes (uint8 in 0..15), nearest, ties to even, saturating at 6.

    The sign bit is copied from the input's sign bit, so -0.0 and small negatives
    that round to zero give code 8.
    """
    y = np.asarray(y, dtype=np.float32)
    mag_code = _round_to_grid(np.abs(y).astype(np.float64), _E2M1_GRID)
    return (mag_code | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def e4m3_encode_satfinite(u: np.ndarray) -> np.ndarray:
    """FP32 values -> E4M3 bytes, nearest, ties to even, finite results only.

    Anything at or beyond 448 in magnitude gives 448 (0x7E / 0xFE); NaN is never
    produced for finite input.
    """
    u = np.asarray(u, dtype=np.float32)
    if not np.all(np.isfinite(u)):
        raise ValueError("e4m3_encode_satfinite: non-finite input")
    mag_code = _round_to_grid(np.abs(u).astype(np.float64), _E4M3_GRID)
    return (mag_code | (np.signbit(u).astype(np.int64) << 7)).astype(np.uint8)


def unpack_fp4(codes: np.ndarray) -> np.ndarray:
    """Packed FP4 bytes [..., K/2] -> codes [..., K]: element 2i is the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = c >> 4
    return out


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Codes [..., K] in 0..15 -> bytes [..., K/2], element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
