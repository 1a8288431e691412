"""moe_forward_fused: RMSNorm of the residual stream before the layer and the residual add
after it, in the layer's own launches, against the oracle (oracle/norm.py).

x is an intermediate the GPU rounds to BF16 from FP32 arithmetic: it must be a correct
rounding of a value within the FP32 error bound of the FP64 RMSNorm (the sum of H squares
in any order is within gamma_H = H u / (1 - H u) of exact, u = 2^-24; the square root,
divide and two multiplies add a few u), i.e. |x_gpu - x64| <= ulp(x64) / 2 + delta |x64|.
The rest of the layer is then checked on the GPU's own x, as the oracle's router and
experts would see it, and the residual stream against r + y_oracle with the output bar
plus half a BF16 ulp of the sum (the single rounding of r + y)."""
import numpy as np
import pytest
import torch

import synth
from oracle import layer as OL
from oracle import norm as N
from oracle.formats import bf16_to_f64
from parity_util import bf16_bits_to_f64, check_ids, device_layer, host_layer, say

pytestmark = pytest.mark.gpu

CASES = [("flint_w4a16", 1), ("flint_w4a16", 8), ("inkling_w4a4", 5), ("tiny_bf16", 3),
         ("mistral_mxfp4_a8", 64), ("mistral_mxfp4_a4", 2)]
EPS = 1e-5


def _bf16_ulp(v):
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def _inputs(name, T):
    cfg = synth.CONFIGS[name]
    rng = np.random.default_rng([77, cfg.cid, T])
    r = synth.to_bf16_bits(rng.normal(size=(T, cfg.H)) * 2.5)
    g = synth.to_bf16_bits(1.0 + 0.1 * rng.normal(size=cfg.H))
    return r, g


@pytest.mark.parametrize("name,T", CASES)
def test_fused_norm_and_residual(lib, name, T):
    say(f"[fused] {name} T={T}")
    dl = device_layer(name)
    cfg = dl.cfg
    L = host_layer(name)
    r_np, g_np = _inputs(name, T)
    r = torch.from_numpy(r_np.view(np.int16)).cuda()
    g = torch.from_numpy(g_np.view(np.int16)).cuda()
    ws = lib.Workspace(dl, T)
    out, x, ids, w, xq = lib.forward_fused(dl, r, g, EPS, ws)
    torch.cuda.synchronize()
    # x: a correct rounding of a value within the FP32 bound of the FP64 RMSNorm
    x64 = N.rms_norm(r_np, g_np, EPS)
    xg = bf16_bits_to_f64(x)
    delta = (cfg.H + 8) * 2.0 ** -24
    assert np.all(np.abs(xg - x64) <= 0.5 * _bf16_ulp(x64) + delta * np.abs(x64)), "x out of bound"
    same_bits = np.mean(x.view(torch.int16).cpu().numpy().view(np.uint16) == N.to_bf16_bits(x64))
    say(f"[fused]   x bits equal to the oracle's rounding: {same_bits:.6f}")
    # the layer on the GPU's own x: the same ids, weights, xq and y as moe_forward
    x_bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    y2, ids2, w2, xq2 = lib.forward(dl, x, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids2.cpu().numpy())
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w2.cpu().numpy().view(np.uint32))
    if xq is not None:
        p1, p2 = lib.split_xq(dl, xq, T), lib.split_xq(dl, xq2, T)
        for key in p1:
            assert np.array_equal(p1[key].cpu().numpy(), p2[key].cpu().numpy()), key
    og = bf16_bits_to_f64(out)
    rv = bf16_to_f64(r_np)
    # resid_out = RNE(r + y32): within one BF16 ulp of the sum of r and the BF16 y
    yb = bf16_bits_to_f64(y2)
    assert np.all(np.abs(og - (rv + yb)) <= _bf16_ulp(rv + yb) + 0.5 * _bf16_ulp(yb) + 1e-30)
    # against the oracle evaluated on the GPU's x
    ref = OL.moe_layer(L, x_bits)
    ids_g = ids.cpu().numpy()
    assert not check_ids(ids_g, ref, cfg.k)
    if np.array_equal(ids_g, ref["ids"]):
        want = N.residual_out(r_np, ref["y"])
        d = og - want
        s = max(1.0, float(np.sqrt(np.mean(ref["y"] ** 2))))
        half = 0.5 * _bf16_ulp(want)
        ok_abs = np.all(np.abs(d) <= 2e-2 * s + half)
        rel = np.linalg.norm(d) / np.linalg.norm(ref["y"])
        rel_bar = 1e-2 + np.linalg.norm(half) / np.linalg.norm(ref["y"])
        say(f"[fused]   resid_out: max |d| / s = {np.max(np.abs(d)) / s:.3g}, rel_l2 {rel:.3g} (bar {rel_bar:.3g})")
        if cfg.afmt == "bf16":
            assert ok_abs and rel <= rel_bar
        else:   # h re-quantized: the oracle's own y may differ by codes FP32 and FP64 h round apart
            assert rel <= max(rel_bar, 2e-2)


def test_fused_in_place(lib):
    name, T = "flint_w4a16", 4
    dl = device_layer(name)
    r_np, g_np = _inputs(name, T)
    r = torch.from_numpy(r_np.view(np.int16)).cuda()
    g = torch.from_numpy(g_np.view(np.int16)).cuda()
    ws = lib.Workspace(dl, T)
    out, x, _, _, _ = lib.forward_fused(dl, r, g, EPS, ws)
    r2 = r.clone()
    lib.forward_fused(dl, r2, g, EPS, ws, resid_out=r2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r2.view(torch.int16))
