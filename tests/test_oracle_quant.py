"""Pins for oracle/quant.py: Four-Over-Six NVFP4 and FP8 per-token quantizers.

The Four-Over-Six rule ("Inkling 2 Small on vLLM: Day-0 Support", mixed-precision MoE
and Four-Over-Six NVFP4): per 16-element block, scale the block maximum to 6 and to 4,
keep the candidate with the lower reconstruction MAE. The checks here rebuild both
candidates independently (brute-force nearest grid values, exact FP64 / rational
reconstruction errors) and compare with the oracle's FP32 emulation.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q

F32 = np.float32


def _row(blocks):
    """A row of 16-element blocks followed by a block holding 2688, so that g = 1."""
    parts = [np.asarray(b, dtype=F32) for b in blocks]
    anchor = np.zeros(16, F32)
    anchor[0] = 2688.0
    return np.concatenate(parts + [anchor])[None, :]


def _decode(codes, sbytes, g):
    return Q.dequant_nvfp4_rows(codes, sbytes, g)


def test_global_scale_is_amax_over_2688():
    x = np.zeros((1, 32), F32)
    x[0, 5] = -13.0
    _, _, g, _ = Q.quantize_nvfp4_4o6(x)
    assert g[0] == F32(13.0) / F32(2688.0)


def test_block_exact_at_four_picks_four():
    blk = np.array([0, 1, 2, 3, 4, -1, -2, -3, -4, 0, 1, 2, 3, 4, 0, 0], F32)
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert g[0] == 1.0
    assert ch[0, 0] == 4
    assert sb[0, 0] == 0x38                     # S4 = 4 / 4 = 1.0
    assert np.array_equal(_decode(codes, sb, g)[0, :16], blk)


def test_block_exact_at_six_picks_six():
    blk = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -6, -4, -3, -2, -1.5, -1, -0.5, 0], F32)
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert ch[0, 0] == 6 and sb[0, 0] == 0x38   # S6 = 6 / 6 = 1.0, error 0
    assert np.array_equal(_decode(codes, sb, g)[0, :16], blk)


def test_all_equal_block_ties_to_six():
    blk = np.full(16, 6.0, F32)                 # both candidates exact (S6 = 1, S4 = 1.5)
    _, sb, _, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert ch[0, 0] == 6 and sb[0, 0] == 0x38


def test_token_max_block_saturates_and_ties_to_six():
    x = np.linspace(-1.0, 1.0, 32).astype(F32) * F32(3.7)
    x[3] = F32(-7.25)                            # the row maximum sits in block 0
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(x[None, :])
    # (a/g)/4 = 672 > 448: the 4-candidate saturates to 448 = the 6-candidate's scale
    assert sb[0, 0] == 0x7E and ch[0, 0] == 6


def test_zero_block_and_zero_row():
    blk = np.zeros(16, F32)
    blk[3] = -0.0
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert sb[0, 0] == 0 and ch[0, 0] == 6
    q = F.unpack_fp4(codes)[0, :16]
    assert q[3] == 8 and np.all(np.delete(q, 3) == 0)
    z = np.zeros((2, 32), F32)
    z[1, 7] = -0.0
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(z)
    assert np.all(g == 0) and np.all(sb == 0) and np.all(ch == 6)
    q = F.unpack_fp4(codes)
    assert q[1, 7] == 8 and q.sum() == 8


def test_scale_underflow_both_candidates():
    blk = np.zeros(16, F32)
    blk[0] = 2.0 ** -12                          # u6, u4 < 2^-10: both scales round to 0
    blk[1] = -(2.0 ** -13)
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert sb[0, 0] == 0 and ch[0, 0] == 6
    q = F.unpack_fp4(codes)[0, :16]
    assert q[0] == 0 and q[1] == 8


def test_scale_underflow_one_candidate_picks_four():
    blk = np.zeros(16, F32)
    blk[0] = 5 * 2.0 ** -10                      # u6 < 2^-10 -> S6 = 0; u4 > 2^-10 -> S4 = 2^-9
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert ch[0, 0] == 4 and sb[0, 0] == 0x01
    # 5*2^-10 / 2^-9 = 2.5 -> E2M1 tie 2 vs 3 -> even code (2.0) -> reconstruction 2^-8
    assert _decode(codes, sb, g)[0, 0] == 2.0 ** -8


# ---------------------------------------------------------------- summation order
# Four-Over-Six compares two FP32 error sums, so the order of the additions is part of
# the quantizer (the pairwise tree (i, i+8), then +4, +2, +1). These pins are worked by
# hand; any other order (sequential, adjacent pairs, reversed) gives different bits.
T24 = 2.0 ** -24          # half an ulp of 1.0: 1 + T24 rounds to 1.0 (tie, even mantissa)


def test_tree_sum16_order_worked_values():
    # [1, T24 x 15]: level 1 gives 1 + T24 -> 1.0 and seven pairs 2*T24; level 2 gives
    # 1 + 2*T24 (exact) and 4*T24 x 3; level 3: 1 + 6*T24 and 8*T24; total 1 + 14*T24.
    # A sequential sum absorbs every T24 into 1.0.
    e = np.full(16, T24, F32)
    e[0] = 1.0
    assert Q.tree_sum16(e) == F32(1.0 + 14 * T24)
    seq = F32(0.0)
    for v in e:
        seq = F32(seq + v)
    assert seq == F32(1.0) and Q.tree_sum16(e) != seq
    # the error vectors of the flip block below: 1 at index 1 (target 6) or index 2
    # (target 4), T24 at indices 6, 9, 10
    e6 = np.zeros(16, F32); e6[1] = 1.0
    e4 = np.zeros(16, F32); e4[2] = 1.0
    for ev in (e6, e4):
        ev[[6, 9, 10]] = T24
    # target 6: (1,9) 1+T24 -> 1; (2,10) T24; (6,14) T24 | +4: s[1] = 1, s[2] = 2*T24 |
    #   +2: s[0] = 2*T24, s[1] = 1 | total 1 + 2*T24 (exact)
    assert Q.tree_sum16(e6) == F32(1.0 + 2 * T24)
    # target 4: (1,9) T24; (2,10) 1+T24 -> 1; (6,14) T24 | +4: s[1] = T24, s[2] = 1+T24 -> 1 |
    #   +2: s[0] = 1, s[1] = T24 | total 1 + T24 -> 1.0
    assert Q.tree_sum16(e4) == F32(1.0)


def test_summation_order_decides_four_over_six():
    """A block whose exact errors tie (6 would win) but whose tree-ordered FP32 errors pick 4.

    g = 1 (anchor 2688), block max 24: S6 = 4 (d6 = 4), S4 = 6 (d4 = 6), both exact.
      24: 24/4 = 6 and 24/6 = 4, exact at both targets.
       3: 3/4 = 0.75 ties 0.5 / 1.0 -> even code (1.0) -> 4, error 1;  3/6 = 0.5 exact.
       4: 4/4 = 1 exact;  4/6 = 0.667 -> 0.5 -> 3, error 1.
     T24 at indices 6, 9, 10: zero codes at both targets, error T24 each.
    Exact sums: both 1 + 3*T24 (a tie, so 6). FP32 sequential: both 1.0 (6). FP32 tree
    (worked above): err6 = 1 + 2*T24 > err4 = 1.0, so the quantizer keeps 4, with scale
    byte E4M3(6) = 0x4C and codes 24 -> 4 (code 6), 3 -> 0.5 (code 1), 4 -> 0.5 (code 1).
    """
    blk = np.zeros(16, F32)
    blk[0], blk[1], blk[2] = 24.0, 3.0, 4.0
    blk[[6, 9, 10]] = T24
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(_row([blk]))
    assert g[0] == 1.0
    assert ch[0, 0] == 4 and sb[0, 0] == 0x4C
    q = F.unpack_fp4(codes)[0, :16]
    assert q[0] == 6 and q[1] == 1 and q[2] == 1 and np.all(q[3:] == 0)


def _nearest_e4m3(u):
    """Brute-force nearest finite E4M3 (non-negative u), ties to the even byte."""
    grid = F.E4M3_TABLE[:0x7F]
    d = np.abs(grid - u)
    c = np.nonzero(d == d.min())[0]
    return int(c[0]) if len(c) == 1 else int(c[c % 2 == 0][0])


def _nearest_code_exact(x, d):
    """argmin over the 16 E2M1 codes of |x - v*d| (exact in FP64 here), ties to even code,
    sign taken from x."""
    mags = np.array(F.E2M1_MAGNITUDES)
    dist = np.abs(abs(x) - mags * d)
    c = np.nonzero(dist == dist.min())[0]
    m = int(c[0]) if len(c) == 1 else int(c[c % 2 == 0][0])
    return m | (8 if np.signbit(x) else 0)


def _bf16_values(lo_exp, hi_exp):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(bits)
    v = v[np.isfinite(v)]
    a = np.abs(v)
    return np.unique(v[(a >= 2.0 ** lo_exp) & (a < 2.0 ** hi_exp)])


@pytest.mark.parametrize("length,lo,hi,stride", [(2, -2, 2, 1), (3, -2, 1, 9)])
def test_exhaustive_short_blocks_exact_decision(length, lo, hi, stride):
    """Every short block over a grid of BF16 values (g = 1): the candidates' scales and
    codes equal brute-force nearest values, and the 4-vs-6 choice equals the choice made
    on exact reconstruction errors (4 only if strictly lower)."""
    vals = _bf16_values(lo, hi)[::stride]
    grids = np.meshgrid(*([vals] * length), indexing="ij")
    combos = np.stack([gr.ravel() for gr in grids], axis=1)
    n = len(combos)
    x = np.zeros((n, 32), F32)
    x[:, :length] = combos
    x[:, 16] = 2688.0
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(x)
    assert np.all(g == 1.0)
    q = F.unpack_fp4(codes)[:, :16]
    rng = np.random.default_rng(7)
    check = rng.choice(n, size=min(n, 3000), replace=False)  # exact rebuild on a sample
    for r in check:
        xb = combos[r]
        m = float(np.max(np.abs(xb)))
        errs, cands = {}, {}
        for c in (6, 4):
            sbyte = _nearest_e4m3(m / c)            # exact m / c here: far from E4M3 midpoints
            S = F.E4M3_TABLE[sbyte]
            if S == 0:
                qs = [8 if np.signbit(v) else 0 for v in xb]
                err = sum(Fraction(abs(float(v))) for v in xb)
            else:
                qs = [_nearest_code_exact(float(v), S) for v in xb]
                err = sum(abs(Fraction(float(v)) - Fraction(F.E2M1_TABLE[cc]) * Fraction(S))
                          for v, cc in zip(xb, qs))
            errs[c], cands[c] = err, (sbyte, qs)
        want = 4 if errs[4] < errs[6] else 6
        assert ch[r, 0] == want, (xb, errs)
        sbyte, qs = cands[want]
        assert sb[r, 0] == sbyte
        assert list(q[r, :length]) == qs
    # the vectorized whole-set check of the decision: FP64 errors are exact for these values
    S6 = F.E4M3_TABLE[np.array([_nearest_e4m3(v) for v in np.max(np.abs(combos), 1) / 6])]
    S4 = F.E4M3_TABLE[np.array([_nearest_e4m3(v) for v in np.max(np.abs(combos), 1) / 4])]

    def exact_err(S):
        mags = np.array(F.E2M1_MAGNITUDES)
        a = np.abs(combos)[:, :, None]
        dist = np.abs(a - mags[None, None, :] * S[:, None, None])
        return np.where(S[:, None] == 0, np.abs(combos), dist.min(axis=2)).sum(axis=1)

    e6, e4 = exact_err(S6), exact_err(S4)
    want = np.where(e4 < e6, 4, 6)
    assert np.array_equal(ch[:, 0], want)


def test_random_blocks_fp32_decision_matches_exact():
    """10^5 random 16-blocks (N(0,1) with 1 % outliers x20, BF16): the FP32 decision equals
    the decision on FP64 reconstruction errors except within 2^-20 relative near-ties."""
    rng = np.random.default_rng(11)
    n = 100_000
    v = rng.normal(size=(n, 16))
    v = np.where(rng.random((n, 16)) < 0.01, 20 * v, v)
    import torch
    v = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).float().numpy()
    x = np.zeros((n, 32), F32)
    x[:, :16] = v
    x[:, 16] = np.max(np.abs(v), axis=1) * F32(1.7)   # varied g, block max below the row max
    codes, sb, g, ch = Q.quantize_nvfp4_4o6(x)
    m = np.max(np.abs(v), axis=1).astype(F32)
    errs = {}
    for c in (6, 4):
        u = (m / g) / F32(c)
        S = np.array([F.E4M3_TABLE[_nearest_e4m3(float(t))] for t in u])
        d = (S.astype(F32) * g).astype(F32).astype(np.float64)
        y = (v / d.astype(F32)[:, None]).astype(F32)      # FP32 quotient, as defined
        qc = F.e2m1_encode(y)
        r = F.E2M1_TABLE[qc] * d[:, None]                 # exact in FP64
        errs[c] = np.abs(v.astype(np.float64) - r).sum(axis=1)
    exact = np.where(errs[4] < errs[6], 4, 6)
    # Exact ties and near-ties can fall either way once the errors are rounded to FP32:
    # the rule is defined on the FP32 sums. Away from them the decisions must agree.
    near = np.abs(errs[4] - errs[6]) < 2.0 ** -20 * errs[6]
    mismatch = (exact != ch[:, 0]) & ~near
    assert mismatch.sum() == 0
    assert near.sum() < n // 100                          # with this seed: 381 of 10^5
    tie = errs[4] == errs[6]
    assert np.mean(ch[tie, 0] == 6) > 0.95                 # exact ties mostly stay ties in FP32
    assert 0.05 < np.mean(ch[:, 0] == 4) < 0.95            # both candidates are used


def test_fp8_token_scale_and_max_code():
    x = np.array([[0.5, -1000.0, 3.0, 0.0, -0.0]], F32)
    codes, s = Q.quantize_fp8_token(x)
    assert s[0] == F32(1000.0) / F32(448.0)
    assert codes[0, 1] == 0xFE                  # -a / s -> -448
    assert codes[0, 3] == 0x00 and codes[0, 4] == 0x80
    z = np.zeros((1, 8), F32)
    z[0, 2] = -0.0
    codes, s = Q.quantize_fp8_token(z)
    assert s[0] == 0 and codes[0, 2] == 0x80 and codes.sum() == 0x80


def test_fp8_token_dequant_worked_values():
    # 0x38 = 0|0111|000 = 1.0 and 0xC0 = 1|1000|000 = -2.0, times s = 2.5
    v = Q.dequant_fp8_token(np.array([[0x38, 0xC0]], np.uint8), np.array([2.5], F32))
    assert np.array_equal(v, [[2.5, -5.0]])
    # 0x7E = 448 and the smallest subnormal 0x01 = 2^-9, per-row scales 0.125 and 4
    v = Q.dequant_fp8_token(np.array([[0x7E, 0x81], [0x01, 0x00]], np.uint8), np.array([0.125, 4.0], F32))
    assert np.array_equal(v, [[56.0, -(2.0 ** -12)], [2.0 ** -7, 0.0]])


def test_fp8_token_exhaustive_bf16_sweep():
    """Every finite BF16 value in a row whose max is 1000: code = nearest E4M3 of x/s."""
    vals = _bf16_values(-40, 9.9)
    vals = vals[np.abs(vals) <= 1000.0]
    x = np.concatenate([vals, [1000.0]]).astype(F32)[None, :]
    codes, s = Q.quantize_fp8_token(x)
    y = (x[0] / s[0]).astype(F32).astype(np.float64)
    grid = F.E4M3_TABLE[:0x7F]
    d = np.abs(np.abs(y)[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    want = np.array([np.nonzero(c)[0][0] if c.sum() == 1 else np.nonzero(c)[0][np.nonzero(c)[0] % 2 == 0][0]
                     for c in cand])
    want = want | (np.signbit(y).astype(np.int64) << 7)
    assert np.array_equal(codes[0].astype(np.int64), want)


def test_weight_dequant_formats():
    # NVFP4: codes 0x21 -> elements (0.5, 1.0); scale 0x38 (1.0) on block 0, 0x40 (2.0) on block 1
    codes = np.full((1, 16), 0x21, np.uint8)
    sc = np.array([[0x38, 0x40]], np.uint8)
    w = Q.dequant_weights("nvfp4", codes, sc, np.float32(0.5))
    assert np.array_equal(w[0, :4], [0.25, 0.5, 0.25, 0.5])
    assert np.array_equal(w[0, 16:20], [0.5, 1.0, 0.5, 1.0])
    # MXFP4: one E8M0 per 32 values
    sc = np.array([[125]], np.uint8)            # 2^-2
    w = Q.dequant_weights("mxfp4", codes, sc, None)
    assert np.array_equal(w[0, :2], [0.125, 0.25]) and w.shape == (1, 32)
    # MXFP8: E4M3 codes with an E8M0 per 32
    c8 = np.full((1, 32), 0x3C, np.uint8)       # 1.5
    w = Q.dequant_weights("mxfp8", c8, np.array([[128]], np.uint8), None)
    assert np.all(w == 3.0)


# ------------------------------------------------------------------ MXFP4 requant
def _mx_decode(packed, sbytes):
    """MXFP4 rows back to FP64 from the format's own tables (E2M1 value times 2^(byte-127))."""
    from oracle.formats import e2m1_value
    c = Q.unpack_fp4(packed).astype(np.int64)
    v = np.vectorize(e2m1_value)(c)
    rows, cols = c.shape
    ex = np.repeat(sbytes.astype(np.int64) - 127, 32, axis=1)
    return np.ldexp(v, ex)


def test_mxfp4_worked_block():
    """amax 7 -> floor(log2 7) = 2 -> exponent 0 (byte 127); 6 -> code 7, 0.1 -> 0,
    -3 -> 13, 7 saturates to 6 (code 7)."""
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [6.0, 0.1, -3.0, 7.0]
    codes, s = Q.quantize_mxfp4(x)
    assert s.tolist() == [[127]]
    assert codes[0, :2].tolist() == [7 | (0 << 4), 13 | (7 << 4)]
    assert np.all(codes[0, 2:] == 0)


def test_mxfp4_round_trip_of_representable_blocks():
    """Blocks built from E2M1 values times 2^X come back bit for bit."""
    from oracle.formats import e2m1_value
    rng = np.random.default_rng(31)
    c = rng.integers(0, 16, size=(20, 256))
    X = rng.integers(-20, 20, size=(20, 8))
    v = np.ldexp(np.vectorize(e2m1_value)(c), np.repeat(X, 32, axis=1)).astype(np.float32)
    codes, s = Q.quantize_mxfp4(v)
    back = _mx_decode(codes, s)
    assert np.array_equal(back, v.astype(np.float64))


def test_mxfp4_scale_is_floor_log2_minus_2_and_error_bounded():
    """The scale byte from math.log2 (another route than frexp), and every element within
    half an E2M1 step of its value, or saturated at 6 when the block exceeds 6 * 2^X."""
    import math
    rng = np.random.default_rng(32)
    x = (rng.normal(size=(16, 512)) * np.exp(rng.normal(size=(16, 1)) * 4)).astype(np.float32)
    codes, s = Q.quantize_mxfp4(x)
    blocks = np.abs(x.reshape(16, -1, 32)).max(axis=2)
    want = np.vectorize(lambda a: min(127, max(-127, math.floor(math.log2(a)) - 2)) + 127)(blocks.astype(np.float64))
    assert np.array_equal(s, want)
    back = _mx_decode(codes, s)
    X = np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    y = np.abs(x.astype(np.float64)) / X
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    bound = np.maximum(half, y - 6.0) * X
    assert np.all(np.abs(back - x) <= bound * (1 + 1e-12))


def test_mxfp4_zero_and_extreme_blocks():
    x = np.zeros((1, 96), np.float32)
    x[0, 5] = -0.0
    x[0, 32] = 2.0 ** -133            # below the E8M0 range: exponent clamps to -127
    x[0, 64] = 3.0e38                 # near the FP32 top: exponent 125
    codes, s = Q.quantize_mxfp4(x)
    assert s.tolist() == [[0, 0, 127 + 125]]
    c = Q.unpack_fp4(codes)[0]
    assert c[5] == 8 and c[0] == 0                  # signed zero kept
    assert c[32] == 0                               # 2^-133 / 2^-127 = 2^-6 rounds to 0
    assert c[64] == 7                               # 3e38 / 2^125 = 7.05 saturates to 6 (code 7)


# ------------------------------------------------------------- NVFP4 weight requant
def test_nvfp4_weights_match_the_activation_quantizer_where_it_picks_6():
    """One tensor of one row is one activation row: the global scale is the same, and on
    every block where Four-Over-Six keeps the 6 candidate the codes and scales agree."""
    rng = np.random.default_rng(51)
    for trial in range(4):
        row = (rng.normal(size=(1, 2048)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        c4, s4, g4, ch = Q.quantize_nvfp4_4o6(row)
        cw, sw, gw = Q.quantize_nvfp4_weights(row[None])
        assert gw[0] == g4[0]
        six = ch[0] == 6
        assert six.sum() > 0
        assert np.array_equal(sw[0, 0][six], s4[0][six])
        cu_w, cu_a = Q.unpack_fp4(cw[0]).reshape(-1, 16), Q.unpack_fp4(c4).reshape(-1, 16)
        assert np.array_equal(cu_w[six], cu_a[six])


def test_nvfp4_weights_worked_tensor():
    """amax 2688 -> g = 1; a block with max 6 takes S = 1 (byte 0x38), exact E2M1 values
    stay exact; a block with max 12 takes S = 2 (byte 0x40)."""
    x = np.zeros((1, 2, 32), np.float32)
    x[0, 0, :4] = [6.0, -3.0, 0.5, 1.5]
    x[0, 0, 16:18] = [12.0, 3.0]
    x[0, 1, 0] = 2688.0
    codes, s, g = Q.quantize_nvfp4_weights(x)
    assert g.tolist() == [1.0]
    assert s[0, 0].tolist() == [0x38, 0x40]
    c = Q.unpack_fp4(codes[0, 0])
    assert c[:4].tolist() == [7, 8 | 5, 1, 3] and c[16:18].tolist() == [7, 3]


def test_nvfp4_weights_zero_tensor_and_error_bound():
    rng = np.random.default_rng(52)
    x = rng.normal(size=(3, 8, 64)).astype(np.float32) * np.array([0.02, 1.0, 5.0], np.float32)[:, None, None]
    x[1] = 0.0
    x[1, 2, 3] = -0.0
    codes, s, g = Q.quantize_nvfp4_weights(x)
    assert g[1] == 0 and np.all(s[1] == 0)
    cz = Q.unpack_fp4(codes[1].reshape(8, 32))
    assert cz[2, 3] == 8 and np.all(np.delete(cz.ravel(), 2 * 64 + 3) == 0)
    for t in (0, 2):
        back = Q.dequant_nvfp4_rows(codes[t], s[t], np.full(8, g[t], np.float32))
        rel = np.linalg.norm(back - x[t]) / np.linalg.norm(x[t])
        assert rel < 0.12, rel


# ------------------------------------------------------------------ MXFP8 requant
def test_mxfp8_worked_block():
    """amax 500 -> floor(log2 500) = 8 -> exponent 0 (byte 127); 448 stays, 500 saturates
    to 448, 0.3 rounds to the nearest E4M3 value 0.3125 (0x2A), -2.0 is 0xC0."""
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [448.0, 500.0, 0.3, -2.0]
    codes, s = Q.quantize_mxfp8(x)
    assert s.tolist() == [[127]]
    assert codes[0, :4].tolist() == [0x7E, 0x7E, 0x2A, 0xC0]
    assert F.e4m3_value(0x2A) == 0.3125


def test_mxfp8_round_trip_of_representable_blocks():
    """Blocks of finite E4M3 values times 2^X whose largest magnitude is 448 * 2^X (so the
    shared exponent is X) come back bit for bit. A block topped by 240 * 2^X instead takes
    exponent X - 1, and 240 * 2 saturates to 448: E4M3 has no 1.875 * 2^8."""
    rng = np.random.default_rng(33)
    b = rng.integers(0, 254, size=(12, 256))
    b = b + (b >= 0x7F)                           # skip the NaN bytes 0x7F, 0xFF
    b[:, ::32] = 0x7E                             # 448 in every block
    X = rng.integers(-30, 30, size=(12, 8))
    v = np.ldexp(np.vectorize(F.e4m3_value)(b), np.repeat(X, 32, axis=1)).astype(np.float32)
    codes, s = Q.quantize_mxfp8(v)
    back = np.ldexp(np.vectorize(F.e4m3_value)(codes.astype(np.int64)), np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(back, v.astype(np.float64))


def test_mxfp8_scale_and_error_bound():
    import math
    rng = np.random.default_rng(34)
    x = (rng.normal(size=(8, 512)) * np.exp(rng.normal(size=(8, 1)) * 4)).astype(np.float32)
    codes, s = Q.quantize_mxfp8(x)
    amax = np.abs(x.reshape(8, -1, 32)).max(axis=2).astype(np.float64)
    want = np.vectorize(lambda a: min(127, max(-127, math.floor(math.log2(a)) - 8)) + 127)(amax)
    assert np.array_equal(s, want)
    X = np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    back = np.vectorize(F.e4m3_value)(codes.astype(np.int64)) * X
    y = np.abs(x.astype(np.float64)) / X
    ulp = np.where(y < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    bound = np.maximum(ulp / 2, y - 448.0) * X
    assert np.all(np.abs(back - x) <= bound * (1 + 1e-12))


def test_mxfp8_block_topped_below_256_saturates_its_top():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 240.0                                # E4M3 0x77, exponent 7
    x[0, 1] = 1.0
    codes, s = Q.quantize_mxfp8(x)
    assert s.tolist() == [[126]]                   # floor(log2 240) - 8 = -1
    assert codes[0, :2].tolist() == [0x7E, 0x40]   # 480 saturates to 448; 2.0 exact


# ---------------------------------------------------------------- block-scaled FP8 input
# "Day 0 support for Mistral Large 4 on vLLM", ROCm implementation details: the loader
# reads block-FP8 expert weights with their block scales and dequantizes each expert to
# BF16 before requantizing it to MXFP4.

def test_fp8_block_worked_values():
    # E4M3 0x38 = 1.0, 0x40 = 2.0, 0xC0 = -2.0, 0x3C = 1.5, 0x01 = 2^-9 (smallest subnormal)
    codes = np.array([[0x38, 0x40, 0xC0, 0x3C, 0x01]], np.uint8)
    bits = Q.dequant_fp8_block(codes, np.array([[0.5]], F32), 128, 128)
    assert [int(b) for b in bits[0]] == [0x3F00, 0x3F80, 0xBF80, 0x3F40, 0x3A80]   # 0.5, 1, -1, 0.75, 2^-10


def test_fp8_block_indexing_against_exact_products():
    # a 5 x 7 matrix in 2 x 3 blocks (ragged last row and column of blocks); power-of-two
    # scales keep every product exact, so each element must equal code value * its own
    # block's scale, worked out here with rationals in explicit loops
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, size=(5, 7)).astype(np.uint8)   # non-negative, no NaN
    codes[codes == 0x7F] = 0x7E
    scales = np.ldexp(1.0, rng.integers(-6, 7, size=(3, 3))).astype(F32)
    got = F.bf16_to_f64(Q.dequant_fp8_block(codes, scales, 2, 3))
    for r in range(5):
        for c in range(7):
            want = Fraction(F.e4m3_value(int(codes[r, c]))) * Fraction(float(scales[r // 2, c // 3]))
            assert Fraction(float(got[r, c])) == want, (r, c)


def test_fp8_block_rounds_to_fp32_before_bf16():
    # code 0x31 = 0.5625 and the FP32 scale with bits 0x3FB238E4: the exact product lies
    # just above the BF16 midpoint 0.783203125 (between 0x3F48 = 0.78125 and 0x3F49 =
    # 0.78515625); its FP32 rounding is that midpoint itself, which BF16 rounds to even
    # (0x3F48). Rounding the exact product straight to BF16 would give 0x3F49 instead.
    s = np.array([[0x3FB238E4]], np.uint32).view(F32)
    exact = Fraction(F.e4m3_value(0x31)) * Fraction(float(s[0, 0]))
    mid = Fraction(0.78125) + Fraction(1, 512)
    assert exact > mid
    assert Fraction(float(F32(float(exact)))) == mid
    bits = Q.dequant_fp8_block(np.array([[0x31]], np.uint8), s, 1, 1)
    assert int(bits[0, 0]) == 0x3F48


def test_fp8_block_to_mxfp4_worked_block():
    # one 32-block of E4M3 3.0 (0x44) with scale 2: BF16 6.0 everywhere, amax 6 ->
    # exponent floor(log2 6) - 2 = 0 (byte 127), elements 6 -> E2M1 code 7
    codes = np.full((1, 32), 0x44, np.uint8)
    packed, sb = Q.requant_fp8_block_mxfp4(codes, np.array([[2.0]], F32), 128, 128)
    assert sb.tolist() == [[127]]
    assert packed.tolist() == [[0x77] * 16]


def test_fp8_block_rejects_bad_scale_shape_and_nan():
    with pytest.raises(ValueError):
        Q.dequant_fp8_block(np.zeros((4, 4), np.uint8), np.ones((1, 1), F32), 2, 2)
    with pytest.raises(ValueError):
        Q.dequant_fp8_block(np.full((1, 1), 0x7F, np.uint8), np.ones((1, 1), F32), 1, 1)
