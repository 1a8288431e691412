"""Pins for oracle/layer.py: closed-form layers built by hand.

Each expert's gate, up and down matrices have exactly one nonzero per row, written
directly as codes and scales of the storage format (so the expected output is a closed
form evaluated by indexing, with no matrix product). This pins the nibble order, the
scale block layout, the global scale, which projection feeds the SiLU, the orientation
of every matrix, the routing weights and the combine.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import layer as OL
from oracle import quant as Q
from oracle.formats import bf16_to_f64

H, I, E = 64, 32, 4
SEL_SCALES = {  # per-row scale choices (code/byte, value)
    "nvfp4": [(0x30, 0.5), (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5)],
    "mxfp4": [(126, 0.5), (127, 1.0), (128, 2.0), (125, 0.25)],
    "mxfp8": [(126, 0.5), (127, 1.0), (128, 2.0), (125, 0.25)],
}
E2M1_CODE = {0.5: 1, 1.0: 2, 2.0: 4, 4.0: 6}
E4M3_CODE = {0.5: 0x30, 1.0: 0x38, 2.0: 0x40, 4.0: 0x48}
BF16_BITS = {0.5: 0x3F00, 1.0: 0x3F80, 2.0: 0x4000, 4.0: 0x4080}


def _selection(fmt, rows, K, rng, gscale):
    """A [rows, K] matrix with one nonzero per row, in storage format ``fmt``.

    Returns (tensor dict, cols, values) with values the exact decoded nonzeros.
    """
    cols = rng.integers(0, K, size=rows)
    mags = rng.choice([0.5, 1.0, 2.0, 4.0], size=rows)
    neg = rng.random(rows) < 0.5
    vals = np.where(neg, -mags, mags).astype(np.float64)
    if fmt == "bf16":
        codes = np.zeros((rows, K), np.uint16)
        for r in range(rows):
            codes[r, cols[r]] = BF16_BITS[mags[r]] | (0x8000 if neg[r] else 0)
        return {"codes": codes, "scales": None, "gscale": None}, cols, vals
    if fmt in ("nvfp4", "mxfp4"):
        blk = 16 if fmt == "nvfp4" else 32
        q = np.zeros((rows, K), np.uint8)
        sc = np.full((rows, K // blk), SEL_SCALES[fmt][1][0], np.uint8)
        for r in range(rows):
            q[r, cols[r]] = E2M1_CODE[mags[r]] | (8 if neg[r] else 0)
            byte, sval = SEL_SCALES[fmt][r % 4]
            sc[r, cols[r] // blk] = byte
            vals[r] *= sval
        codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        if fmt == "nvfp4":
            vals *= float(gscale)
        return {"codes": codes, "scales": sc,
                "gscale": np.float32(gscale) if fmt == "nvfp4" else None}, cols, vals
    if fmt == "mxfp8":
        q = np.zeros((rows, K), np.uint8)
        sc = np.full((rows, K // 32), 127, np.uint8)
        for r in range(rows):
            q[r, cols[r]] = E4M3_CODE[mags[r]] | (0x80 if neg[r] else 0)
            byte, sval = SEL_SCALES[fmt][r % 4]
            sc[r, cols[r] // 32] = byte
            vals[r] *= sval
        return {"codes": q, "scales": sc, "gscale": None}, cols, vals
    raise ValueError(fmt)


def _expert(fmt, rng, I_):
    g, pg, cg = _selection(fmt, I_, H, rng, 0.5)
    u, pu, cu = _selection(fmt, I_, H, rng, 0.25)
    d, pd, cd = _selection(fmt, H, I_, rng, 2.0)
    w13 = {"codes": np.concatenate([g["codes"], u["codes"]]),
           "scales": None if g["scales"] is None else np.concatenate([g["scales"], u["scales"]]),
           "gscale": None if g["gscale"] is None else np.array([g["gscale"], u["gscale"]], np.float32)}
    w2 = {"codes": d["codes"], "scales": d["scales"],
          "gscale": None if d["gscale"] is None else np.array([d["gscale"]], np.float32)}
    closed = {"pg": pg, "cg": cg, "pu": pu, "cu": cu, "pd": pd, "cd": cd}
    return w13, w2, closed


def _stack(ts):
    return {k: None if ts[0][k] is None else np.stack([t[k] for t in ts]) for k in ts[0]}


def _build(fmt, shared_fmt, afmt, n_experts, k, seed=0):
    rng = np.random.default_rng(seed)
    cfg = dataclasses.replace(synth.CONFIGS["tiny_bf16"], name="closed", H=H, I=I, E=n_experts,
                              k=k, has_shared=shared_fmt is not None, wfmt=fmt,
                              shared_wfmt=shared_fmt or fmt, afmt=afmt)
    ex = [_expert(fmt, rng, I) for _ in range(n_experts)]
    layer = {"cfg": cfg, "expert_ids": list(range(n_experts)),
             "router_w": np.zeros((n_experts, H), np.float32), "router_bias": None,
             "w13": _stack([e[0] for e in ex]), "w2": _stack([e[1] for e in ex]),
             "sh13": None, "sh2": None}
    closed = [e[2] for e in ex]
    shared = None
    if shared_fmt is not None:
        s13, s2, shared = _expert(shared_fmt, rng, I)
        layer["sh13"] = {kk: None if v is None else v[None] for kk, v in s13.items()}
        layer["sh2"] = {kk: None if v is None else v[None] for kk, v in s2.items()}
    return layer, closed, shared


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _closed_h(c, xv):
    """SwiGLU output of a selection expert, by indexing: h_i = silu(cg_i x[pg_i]) cu_i x[pu_i]."""
    return _silu(c["cg"] * xv[c["pg"]]) * (c["cu"] * xv[c["pu"]])


def _closed_down(c, hv):
    return c["cd"] * hv[c["pd"]]


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "mxfp4", "mxfp8"])
def test_uniform_router_gives_mean_of_experts_plus_shared(fmt):
    layer, closed, shared = _build(fmt, "bf16", "bf16", E, E)
    x = synth.to_bf16_bits(np.random.default_rng(1).normal(size=(3, H)))
    out = OL.moe_layer(layer, x)
    xv = bf16_to_f64(x)
    for t in range(3):
        assert list(out["ids"][t]) == [0, 1, 2, 3]          # all-zero logits: index order
        assert np.all(out["w"][t] == 0.25)
        want = sum(_closed_down(c, _closed_h(c, xv[t])) for c in closed) / E
        want = want + _closed_down(shared, _closed_h(shared, xv[t]))
        assert np.allclose(out["y"][t], want, rtol=1e-13, atol=1e-15)
        for j, c in enumerate(closed):
            assert np.allclose(out["h"][t, j], _closed_h(c, xv[t]), rtol=1e-13, atol=1e-15)


def test_single_expert_plus_shared():
    layer, closed, shared = _build("nvfp4", "nvfp4", "bf16", 1, 1, seed=4)
    x = synth.to_bf16_bits(np.random.default_rng(2).normal(size=(2, H)))
    out = OL.moe_layer(layer, x)
    xv = bf16_to_f64(x)
    for t in range(2):
        assert out["w"][t, 0] == 1.0
        want = _closed_down(closed[0], _closed_h(closed[0], xv[t])) + \
            _closed_down(shared, _closed_h(shared, xv[t]))
        assert np.allclose(out["y"][t], want, rtol=1e-13, atol=1e-15)


def _mx_decode(codes, scales, elem):
    """MX rows by hand: E2M1 nibbles (element 2i low) or E4M3 bytes, times 2^(byte - 127)
    of each 32-block's E8M0 scale."""
    from oracle import formats as F
    if elem == "fp4":
        q = np.stack([codes & 0x0F, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
        v = np.array([F.e2m1_value(int(c)) for c in range(16)])[q]
    else:
        v = np.array([F.e4m3_value(int(b)) for b in range(256)])[codes]
    return v * np.repeat(2.0 ** (scales.astype(np.float64) - 127.0), 32, axis=-1)


WFMT_OF = {"nvfp4_4o6": "nvfp4", "fp8_token": "mxfp4", "mxfp4": "mxfp4", "mxfp8": "mxfp8"}


def _quant_dequant(afmt, v32):
    if afmt == "nvfp4_4o6":
        c_, s_, g_, _ = Q.quantize_nvfp4_4o6(v32)
        return Q.dequant_nvfp4_rows(c_, s_, g_)[0]
    if afmt == "fp8_token":
        c_, s_ = Q.quantize_fp8_token(v32)
        return Q.dequant_fp8_token(c_, s_)[0]
    c_, s_ = (Q.quantize_mxfp4 if afmt == "mxfp4" else Q.quantize_mxfp8)(v32)
    return _mx_decode(c_, s_, "fp4" if afmt == "mxfp4" else "fp8")[0]


@pytest.mark.parametrize("afmt", ["nvfp4_4o6", "fp8_token", "mxfp4", "mxfp8"])
def test_quantized_activations_feed_both_projections(afmt):
    """Routed experts see quantize(x) before gate/up and quantize(h) before down; the
    shared expert sees BF16 x and an unquantized h. MX formats: MXFP4 activations (a4w4)
    on MXFP4 experts, MXFP8 activations on MXFP8 experts."""
    layer, closed, shared = _build(WFMT_OF[afmt], "bf16", afmt, E, E, seed=6)
    x = synth.to_bf16_bits(np.random.default_rng(3).normal(size=(2, H)) * 3)
    out = OL.moe_layer(layer, x)
    xv = bf16_to_f64(x)
    for t in range(2):
        x32 = xv[t:t + 1].astype(np.float32)
        xhat = _quant_dequant(afmt, x32)
        assert not np.array_equal(xhat, xv[t])            # the quantization is not a no-op
        want = np.zeros(H)
        for c in closed:
            h = _closed_h(c, xhat)[None].astype(np.float32)
            hhat = _quant_dequant(afmt, h)
            want += 0.25 * _closed_down(c, hhat)
        want += _closed_down(shared, _closed_h(shared, xv[t]))
        assert np.allclose(out["y"][t], want, rtol=1e-12, atol=1e-14)


def test_bf16_layer_matches_torch_float64():
    """A random BF16 layer against torch's own float64 matmul and SiLU."""
    cfg = synth.CONFIGS["tiny_bf16"]
    L = synth.make_layer(cfg)
    x = synth.make_x(cfg, 1)
    out = OL.moe_layer(L, x)
    xt = torch.from_numpy(bf16_to_f64(x))

    def mlp(t13, t2, pos):
        W13 = torch.from_numpy(bf16_to_f64(t13["codes"][pos]))
        W2 = torch.from_numpy(bf16_to_f64(t2["codes"][pos]))
        gu = xt @ W13.T
        return (torch.nn.functional.silu(gu[:, :cfg.I]) * gu[:, cfg.I:]) @ W2.T

    want = sum(out["w"][0, j] * mlp(L["w13"], L["w2"], int(out["ids"][0, j])) for j in range(cfg.k))
    want = want + mlp(L["sh13"], L["sh2"], 0)
    assert np.allclose(out["y"], want.numpy(), rtol=1e-12, atol=1e-15)
