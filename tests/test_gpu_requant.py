"""GPU parity of the load-time requantizers: moe_requant_mxfp4 (codes and E8M0 scales)
and moe_requant_nvfp4 (codes, E4M3 scales and tensor scales) bit-exact against the
oracle on the same BF16 inputs, and layers built from their output against the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant as OQ
from parity_util import bf16_bits_to_f64, say

pytestmark = pytest.mark.gpu


def _check(lib, xb):
    say(f"[requant] mxfp4 rows={xb.shape[0]} cols={xb.shape[1]}")
    codes, scales = lib.requant_mxfp4(torch.from_numpy(xb.view(np.int16)).cuda())
    torch.cuda.synchronize()
    x32 = bf16_bits_to_f64(torch.from_numpy(xb.view(np.int16))).astype(np.float32)
    rc, rs = OQ.quantize_mxfp4(x32)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_requant_mxfp4_wide_range_rows(lib):
    rng = np.random.default_rng(41)
    x = rng.normal(size=(64, 2048)) * np.exp(rng.normal(size=(64, 1)) * 6)
    _check(lib, synth.to_bf16_bits(x))


def test_requant_mxfp4_ragged_grid(lib):
    """300 x 96: 900 blocks, not a multiple of the 256-thread launch."""
    rng = np.random.default_rng(42)
    _check(lib, synth.to_bf16_bits(rng.normal(size=(300, 96)) * 0.02))


def test_requant_mxfp4_special_blocks(lib):
    rows = np.zeros((6, 64))
    rows[0, 3] = -0.0
    rows[1, :32] = 2.0 ** -133                     # BF16 subnormal: exponent clamps to -127
    rows[2, :32] = 3.0e38                          # exponent 125, values saturate
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    rows[3, :8] = ties                              # amax 6: exponent 0, every tie of E2M1
    rows[3, 8:16] = -ties
    rows[4, :8] = ties * 2.0 ** -10                 # the same ties, scaled
    rows[5, :32] = np.linspace(-7.9, 7.9, 32)       # amax 7.9: exponent 0, saturation at 6
    xb = synth.to_bf16_bits(rows)
    xb[0, 3] = 0x8000                               # an exact -0
    _check(lib, xb)


def test_requant_mxfp4_all_bf16_values(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    bits = bits[np.isfinite(v)]
    n = len(bits) // 2048 * 2048
    _check(lib, bits[:n].reshape(-1, 2048).copy())


def test_requantized_layer_runs_end_to_end(lib):
    """The load path end to end: a Flint-shaped BF16 layer (16 experts, top-4, BF16
    shared expert) has its routed experts requantized to MXFP4 on the GPU, the codes are
    loaded as an MXFP4 layer, and moe_forward's ids and y match the oracle evaluated on
    those same codes."""
    import dataclasses
    from oracle import layer as OL
    from parity_util import check_ids, y_close
    base = dataclasses.replace(synth.CONFIGS["flint_bf16"], name="flint_bf16_e16", E=16, k=4,
                               router_bias=False)
    L = synth.make_layer(base)
    cfg = dataclasses.replace(base, name="flint_mxfp4_requant", wfmt=synth.W_MXFP4)
    Lq = dict(L, cfg=cfg)
    for name in ("w13", "w2"):
        c = L[name]["codes"]                                   # BF16 bits [E][rows][K]
        say(f"[requant] layer {name} {c.shape}")
        codes, scales = lib.requant_mxfp4(torch.from_numpy(c.reshape(-1, c.shape[2]).view(np.int16)).cuda())
        torch.cuda.synchronize()
        Lq[name] = {"codes": codes.cpu().numpy().reshape(c.shape[0], c.shape[1], -1),
                    "scales": scales.cpu().numpy().reshape(c.shape[0], c.shape[1], -1), "gscale": None}
    dl = lib.DeviceLayer.from_host(Lq)
    for T in (1, 8):
        x_np = synth.make_x(base, T)
        ref = OL.moe_layer(Lq, x_np)
        ws = lib.Workspace(dl, T)
        y, ids, w, _ = lib.forward(dl, torch.from_numpy(x_np.view(np.int16)).cuda(), ws)
        torch.cuda.synchronize()
        ids_g = ids.cpu().numpy()
        assert not check_ids(ids_g, ref, cfg.k)
        if np.array_equal(ids_g, ref["ids"]):
            ok, max_abs, rel = y_close(bf16_bits_to_f64(y), ref["y"])
            say(f"[requant]   T={T} y max_abs/r={max_abs:.3g} rel_l2={rel:.3g}")
            assert ok, (max_abs, rel)


def _check_nv(lib, x32):
    """x32 [n, rows, cols] FP32 values that are exact BF16."""
    n, rows, cols = x32.shape
    say(f"[requant] nvfp4 tensors={n} rows={rows} cols={cols}")
    xb = synth.to_bf16_bits(x32)
    codes, scales, g = lib.requant_nvfp4(torch.from_numpy(xb.view(np.int16)).cuda())
    torch.cuda.synchronize()
    rc, rs, rg = OQ.quantize_nvfp4_weights(bf16_bits_to_f64(torch.from_numpy(xb.view(np.int16))).astype(np.float32))
    assert np.array_equal(g.cpu().numpy().view(np.uint32), rg.view(np.uint32))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_requant_nvfp4_tensors(lib):
    """Tensors of very different ranges, one of them all zero (with a -0), one with an
    outlier that pushes small blocks' scales into E4M3 subnormals and to zero."""
    rng = np.random.default_rng(61)
    x = rng.normal(size=(5, 40, 256)) * np.array([0.02, 1.0, 300.0, 0.0, 1e-3])[:, None, None]
    x[3] = 0.0
    x[4, 0, 0] = 1e4
    _check_nv(lib, x)


def test_requant_nvfp4_multi_chunk_tensors(lib):
    """Tensors of 300 x 256 = 76800 elements span three reduction chunks of 32768 (the last
    one ragged, 11264 elements). Each tensor's maximum sits in a different chunk (the last,
    the middle, the first), so a tensor scale taken from one chunk only, or one that drops
    the ragged chunk, changes g and every code."""
    rng = np.random.default_rng(62)
    x = rng.normal(size=(3, 300, 256)) * 0.02
    x[0, 297, 5] = -7.5          # element 76037: chunk 2 (the ragged one)
    x[1, 150, 200] = 3.25        # element 38600: chunk 1
    x[2, 3, 9] = 11.0            # element 777: chunk 0
    _check_nv(lib, x)


def test_requant_nvfp4_all_bf16_values(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    n = len(v) // 4096 * 4096
    _check_nv(lib, v[:n].reshape(-1, 1, 4096).copy().astype(np.float64))


def test_nvfp4_requantized_layer_runs_end_to_end(lib):
    """A Flint-shaped BF16 layer (16 experts, top-4, BF16 shared expert) with its routed
    experts requantized to NVFP4 on the GPU (gate, up and down as separate tensors) runs
    through moe_forward; ids and y match the oracle on the same codes and scales."""
    import dataclasses
    from oracle import layer as OL
    from parity_util import check_ids, y_close
    base = dataclasses.replace(synth.CONFIGS["flint_bf16"], name="flint_bf16_e16", E=16, k=4,
                               router_bias=False)
    L = synth.make_layer(base)
    cfg = dataclasses.replace(base, name="flint_nvfp4_requant", wfmt=synth.W_NVFP4)
    Lq = dict(L, cfg=cfg)
    for name, parts in (("w13", 2), ("w2", 1)):
        c = L[name]["codes"]                                      # BF16 bits [E][rows][K]
        E, R, K = c.shape
        say(f"[requant] layer {name} {c.shape}")
        codes, scales, g = lib.requant_nvfp4(torch.from_numpy(c.reshape(E * parts, R // parts, K).view(np.int16)).cuda())
        torch.cuda.synchronize()
        # the whole stack (tensors of 768 x 2048 = 48 chunks each) bit-exact against the oracle
        rc, rs, rg = OQ.quantize_nvfp4_weights(
            bf16_bits_to_f64(torch.from_numpy(c.reshape(E * parts, R // parts, K).view(np.int16))).astype(np.float32))
        assert np.array_equal(g.cpu().numpy().view(np.uint32), rg.view(np.uint32))
        assert np.array_equal(scales.cpu().numpy(), rs)
        assert np.array_equal(codes.cpu().numpy(), rc)
        Lq[name] = {"codes": codes.cpu().numpy().reshape(E, R, K // 2),
                    "scales": scales.cpu().numpy().reshape(E, R, K // 16),
                    "gscale": g.cpu().numpy().reshape(E, parts)}
    dl = lib.DeviceLayer.from_host(Lq)
    for T in (1, 8):
        x_np = synth.make_x(base, T)
        ref = OL.moe_layer(Lq, x_np)
        ws = lib.Workspace(dl, T)
        y, ids, w, _ = lib.forward(dl, torch.from_numpy(x_np.view(np.int16)).cuda(), ws)
        torch.cuda.synchronize()
        ids_g = ids.cpu().numpy()
        assert not check_ids(ids_g, ref, cfg.k)
        if np.array_equal(ids_g, ref["ids"]):
            ok, max_abs, rel = y_close(bf16_bits_to_f64(y), ref["y"])
            say(f"[requant]   T={T} y max_abs/r={max_abs:.3g} rel_l2={rel:.3g}")
            assert ok, (max_abs, rel)


def _check_mx8(lib, xb):
    say(f"[requant] mxfp8 rows={xb.shape[0]} cols={xb.shape[1]}")
    codes, scales = lib.requant_mxfp8(torch.from_numpy(xb.view(np.int16)).cuda())
    torch.cuda.synchronize()
    x32 = bf16_bits_to_f64(torch.from_numpy(xb.view(np.int16))).astype(np.float32)
    rc, rs = OQ.quantize_mxfp8(x32)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_requant_mxfp8_rows(lib):
    rng = np.random.default_rng(71)
    _check_mx8(lib, synth.to_bf16_bits(rng.normal(size=(64, 2048)) * np.exp(rng.normal(size=(64, 1)) * 6)))
    _check_mx8(lib, synth.to_bf16_bits(rng.normal(size=(300, 96)) * 0.02))
    rows = np.zeros((3, 64))
    rows[0, :4] = [448.0, 500.0, 0.3, -2.0]
    rows[1, :32] = 2.0 ** -133
    rows[2, :32] = 3.0e38
    xb = synth.to_bf16_bits(rows)
    xb[0, 10] = 0x8000
    _check_mx8(lib, xb)


def test_requant_mxfp8_all_bf16_values(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    bits = bits[np.isfinite(v)]
    n = len(bits) // 2048 * 2048
    _check_mx8(lib, bits[:n].reshape(-1, 2048).copy())


def test_mxfp8_requantized_layer_runs_end_to_end(lib):
    """A Flint-shaped BF16 layer (16 experts, top-4, BF16 shared expert) requantized to
    MXFP8 on the GPU runs through moe_forward against the oracle on the same codes."""
    import dataclasses
    from oracle import layer as OL
    from parity_util import check_ids, y_close
    base = dataclasses.replace(synth.CONFIGS["flint_bf16"], name="flint_bf16_e16", E=16, k=4,
                               router_bias=False)
    L = synth.make_layer(base)
    cfg = dataclasses.replace(base, name="flint_mxfp8_requant", wfmt=synth.W_MXFP8)
    Lq = dict(L, cfg=cfg)
    for name in ("w13", "w2"):
        c = L[name]["codes"]
        say(f"[requant] layer {name} {c.shape} -> mxfp8")
        codes, scales = lib.requant_mxfp8(torch.from_numpy(c.reshape(-1, c.shape[2]).view(np.int16)).cuda())
        torch.cuda.synchronize()
        Lq[name] = {"codes": codes.cpu().numpy().reshape(c.shape),
                    "scales": scales.cpu().numpy().reshape(c.shape[0], c.shape[1], -1), "gscale": None}
    dl = lib.DeviceLayer.from_host(Lq)
    for T in (1, 8):
        x_np = synth.make_x(base, T)
        ref = OL.moe_layer(Lq, x_np)
        ws = lib.Workspace(dl, T)
        y, ids, w, _ = lib.forward(dl, torch.from_numpy(x_np.view(np.int16)).cuda(), ws)
        torch.cuda.synchronize()
        ids_g = ids.cpu().numpy()
        assert not check_ids(ids_g, ref, cfg.k)
        if np.array_equal(ids_g, ref["ids"]):
            ok, max_abs, rel = y_close(bf16_bits_to_f64(y), ref["y"])
            say(f"[requant]   T={T} y max_abs/r={max_abs:.3g} rel_l2={rel:.3g}")
            assert ok, (max_abs, rel)


# ---------------------------------------------------------------- block-scaled FP8 input
def _check_fp8b(lib, codes, bscale, br, bc):
    rows, cols = codes.shape
    say(f"[requant] fp8-block -> mxfp4 rows={rows} cols={cols} block={br}x{bc}")
    gc, gs = lib.requant_fp8_block_mxfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(bscale).cuda(), br, bc)
    torch.cuda.synchronize()
    rc, rs = OQ.requant_fp8_block_mxfp4(codes, bscale, br, bc)
    assert np.array_equal(gs.cpu().numpy(), rs)
    assert np.array_equal(gc.cpu().numpy(), rc)


def _fp8_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01          # no NaN codes
    return c


def test_requant_fp8_block_128x128(lib):
    rng = np.random.default_rng(51)
    codes = _fp8_codes(rng, (256, 512))
    bscale = np.exp(rng.normal(size=(2, 4)) * 3).astype(np.float32) * 1e-3
    _check_fp8b(lib, codes, bscale, 128, 128)


def test_requant_fp8_block_ragged_and_straddling_blocks(lib):
    """300 x 96 in 128 x 128 blocks (ragged edge blocks), then 45 x 160 in 7 x 48 blocks:
    a 32-block of a row straddles two scale blocks."""
    rng = np.random.default_rng(52)
    codes = _fp8_codes(rng, (300, 96))
    _check_fp8b(lib, codes, (rng.random((3, 1)) + 0.5).astype(np.float32), 128, 128)
    codes = _fp8_codes(rng, (45, 160))
    _check_fp8b(lib, codes, np.exp(rng.normal(size=(7, 4)) * 2).astype(np.float32), 7, 48)


def test_requant_fp8_block_every_code_and_double_rounding(lib):
    """Every finite E4M3 code in every column position, under scales that include the one
    whose products round to FP32 exactly on a BF16 tie (bits 0x3FB238E4)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F] + [0x00, 0x80], np.uint8)   # 256
    codes = np.stack([np.roll(finite, 37 * i) for i in range(32)])                              # [32][256]
    sbits = np.array([0x3FB238E4, 0x3F800000, 0x3B800000, 0x42F00000], np.uint32)
    bscale = np.resize(sbits, (32, 8)).view(np.float32).copy()
    _check_fp8b(lib, codes, bscale, 1, 32)


def test_fp8_block_requantized_layer_runs_end_to_end(lib):
    """The load path from a block-FP8 checkpoint: a 16-expert Flint-shaped layer whose BF16
    expert weights are turned into FP8 with 128 x 128 block scales (amax / 448 per block),
    requantized to MXFP4 on the GPU (codes bit-exact against the oracle), loaded as an
    MXFP4 layer, and run: ids and y against the oracle on those codes."""
    import dataclasses
    from oracle import formats as OF
    from oracle import layer as OL
    from parity_util import check_ids, y_close
    base = dataclasses.replace(synth.CONFIGS["flint_bf16"], name="flint_bf16_e16", E=16, k=4,
                               router_bias=False)
    L = synth.make_layer(base)
    cfg = dataclasses.replace(base, name="flint_mxfp4_from_fp8", wfmt=synth.W_MXFP4)
    Lq = dict(L, cfg=cfg)
    for name in ("w13", "w2"):
        w = bf16_bits_to_f64(torch.from_numpy(L[name]["codes"].view(np.int16)))     # [E][rows][K]
        E, rows, K = w.shape
        w2 = w.reshape(E * rows, K)
        br, bc = 128, 128
        nb_r, nb_c = -(-E * rows // br), -(-K // bc)
        pad = np.zeros((nb_r * br, nb_c * bc))
        pad[:E * rows, :K] = np.abs(w2)
        amax = pad.reshape(nb_r, br, nb_c, bc).max(axis=(1, 3))
        bscale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
        per = bscale[(np.arange(E * rows) // br)[:, None], (np.arange(K) // bc)[None, :]].astype(np.float64)
        fp8 = OF.e4m3_encode_satfinite((w2 / per).astype(np.float32))
        _check_fp8b(lib, fp8, bscale, br, bc)
        codes, scales = lib.requant_fp8_block_mxfp4(torch.from_numpy(fp8).cuda(), torch.from_numpy(bscale).cuda(),
                                                    br, bc)
        torch.cuda.synchronize()
        Lq[name] = {"codes": codes.cpu().numpy().reshape(E, rows, -1),
                    "scales": scales.cpu().numpy().reshape(E, rows, -1), "gscale": None}
    dl = lib.DeviceLayer.from_host(Lq)
    for T in (1, 8):
        x_np = synth.make_x(base, T)
        ref = OL.moe_layer(Lq, x_np)
        ws = lib.Workspace(dl, T)
        y, ids, w, _ = lib.forward(dl, torch.from_numpy(x_np.view(np.int16)).cuda(), ws)
        torch.cuda.synchronize()
        ids_g = ids.cpu().numpy()
        assert not check_ids(ids_g, ref, cfg.k)
        if np.array_equal(ids_g, ref["ids"]):
            ok, max_abs, rel = y_close(bf16_bits_to_f64(y), ref["y"])
            say(f"[requant]   T={T} y max_abs/r={max_abs:.3g} rel_l2={rel:.3g}")
            assert ok, (max_abs, rel)
