"""Pins for oracle/formats.py: hand-worked tables, library decoders, brute force."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_hand_table():
    rows = _read_golden("e2m1_table.txt")
    assert len(rows) == 16
    for r in rows:
        code, value = int(r[0]), float(r[4])
        assert _same(F.E2M1_TABLE[code], value), (code, F.E2M1_TABLE[code], value)


def test_e4m3_hand_spots():
    for r in _read_golden("e4m3_spot.txt"):
        b, v = int(r[0], 16), float(r[1])
        assert _same(F.E4M3_TABLE[b], v), (hex(b), F.E4M3_TABLE[b], v)


def test_e8m0_hand_spots():
    for r in _read_golden("e8m0_spot.txt"):
        b, v = int(r[0], 16), float(r[1])
        assert _same(F.E8M0_TABLE[b], v), (hex(b), F.E8M0_TABLE[b], v)


def test_e4m3_matches_torch_decoder():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    for b in range(256):
        assert _same(F.E4M3_TABLE[b], lib[b]), hex(b)


def test_e8m0_matches_torch_decoder():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().double().numpy()
    for b in range(255):
        assert F.E8M0_TABLE[b] == lib[b], b
    assert math.isnan(F.E8M0_TABLE[255])


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = F.bf16_to_f64(bits)
    fin = np.isfinite(lib)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(lib))


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(bits)
    return v[np.isfinite(v)]


def _brute_nearest(values, grid_vals, grid_codes):
    """Nearest grid value by exhaustive distance; ties to the even code."""
    d = np.abs(values[:, None] - grid_vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    out = np.empty(len(values), dtype=np.int64)
    for i in range(len(values)):
        cs = grid_codes[cand[i]]
        if len(cs) > 1:
            # float64 distances may have rounded (huge inputs): redo them exactly
            x = Fraction(float(values[i]))
            dist = [abs(x - Fraction(float(grid_vals[np.where(grid_codes == c)[0][0]])))
                    for c in cs]
            best = min(dist)
            cs = np.array([c for c, dd in zip(cs, dist) if dd == best])
        if len(cs) == 1:
            out[i] = cs[0]
        else:
            assert len(cs) == 2
            out[i] = cs[cs % 2 == 0][0]
    return out


def test_e2m1_encoder_exhaustive_bf16():
    v = _all_bf16_finite()
    got = F.e2m1_encode(v.astype(np.float32)).astype(np.int64)
    mags = np.array(F.E2M1_MAGNITUDES)
    want = _brute_nearest(np.abs(v), mags, np.arange(8)) | (np.signbit(v).astype(np.int64) << 3)
    assert np.array_equal(got, want)


def test_e2m1_encoder_boundaries():
    # the rounding table: <=0.25 -> 0, (0.25,0.75) -> 0.5, [0.75,1.25] -> 1, (1.25,1.75) -> 1.5,
    # [1.75,2.5] -> 2, (2.5,3.5) -> 3, [3.5,5] -> 4, >5 -> 6
    cases = [(0.25, 0), (0.2500001, 1), (0.75, 2), (1.25, 2), (1.2500001, 3), (1.75, 4),
             (2.5, 4), (2.5000002, 5), (3.5, 6), (5.0, 6), (5.0000005, 7), (1e30, 7),
             (-0.0, 8), (-0.1, 8), (-6.5, 15)]
    for y, code in cases:
        assert F.e2m1_encode(np.float32(y)) == code, (y, code)


def test_e4m3_encoder_exhaustive_bf16():
    v = _all_bf16_finite()
    got = F.e4m3_encode_satfinite(v.astype(np.float32)).astype(np.int64)
    grid = F.E4M3_TABLE[:0x7F]
    want = _brute_nearest(np.abs(v), grid, np.arange(0x7F)) | (np.signbit(v).astype(np.int64) << 7)
    assert np.array_equal(got, want)


def test_e4m3_encoder_matches_torch_cast_below_464():
    # torch's float8_e4m3fn cast is round-to-nearest-even; it gives NaN from 464 upward
    # instead of saturating, so compare only below that.
    v = _all_bf16_finite()
    v = v[np.abs(v) < 464]
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_satfinite(v.astype(np.float32))
    assert np.array_equal(got, lib)


def test_e4m3_encoder_saturates_and_underflows():
    enc = F.e4m3_encode_satfinite
    assert enc(np.float32(448.0)) == 0x7E
    assert enc(np.float32(463.9)) == 0x7E
    assert enc(np.float32(464.0)) == 0x7E          # tie between 448 and the NaN slot -> 448
    assert enc(np.float32(1e20)) == 0x7E
    assert enc(np.float32(-1e20)) == 0xFE
    assert enc(np.float32(2.0 ** -10)) == 0x00     # exactly half the smallest subnormal: even
    assert enc(np.float32(2.0 ** -10 * 1.0000001)) == 0x01
    assert enc(np.float32(7.5 * 2.0 ** -9)) == 0x08  # tie 7 vs 8 subnormal steps -> even (normal)
    with pytest.raises(ValueError):
        enc(np.float32(np.inf))


def test_fp4_pack_roundtrip_and_nibble_order():
    codes = np.arange(16, dtype=np.uint8)
    packed = F.pack_fp4(codes)
    assert packed[0] == 0x10            # element 0 in the low nibble, element 1 in the high
    assert np.array_equal(F.unpack_fp4(packed), codes)
