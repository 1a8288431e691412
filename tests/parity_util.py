"""Helpers shared by the GPU parity tests: cached layers, oracle runs, tolerance checks.

The layer-output bar: with r = max(1, rms(y_oracle)), max |y_gpu - y_oracle| / r <= 2e-2
and ||y_gpu - y_oracle|| / ||y_oracle|| <= 1e-2. Dividing by r changes nothing for layers
whose output rms is below 1; it makes the bar scale-free for the MXFP4 layer, whose
literal exponent range gives outputs of rms ~2e3, where BF16 output rounding alone is
larger than any fixed absolute bound.
"""
from __future__ import annotations

import functools
import sys

import numpy as np

import synth
from oracle import layer as OL
from oracle import router as OR

MAX_ABS = 2e-2
REL_L2 = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def host_layer(name: str):
    say(f"[parity] drawing layer {name}")
    return synth.make_layer(name)


_device_cache = {}


def device_layer(name: str):
    import block_scaled_bit_fp32_amd as moe
    if name not in _device_cache:
        _device_cache.clear()
        import torch
        torch.cuda.empty_cache()
        L = host_layer(name)
        say(f"[parity] uploading layer {name}")
        _device_cache[name] = moe.DeviceLayer.from_host(L)
    return _device_cache[name]


def y_close(y_gpu: np.ndarray, y_ref: np.ndarray):
    """(ok, max_abs_normalized, rel_l2) under the layer-output bar."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return True, 0.0, 0.0
    r = max(1.0, float(np.sqrt(np.mean(y_ref ** 2))))
    d = y_gpu - y_ref
    max_abs = float(np.max(np.abs(d))) / r
    nref = float(np.linalg.norm(y_ref))
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    return (max_abs <= MAX_ABS and rel <= REL_L2), max_abs, rel


def check_ids(ids_gpu: np.ndarray, ref: dict, k: int):
    """Bit-exact top-k ids, except tokens the oracle flags as near-ties, where the GPU's
    set must consist of experts whose FP64 logit is within the tie tolerance of the
    oracle's k-th largest."""
    ids_ref, lg, amb = ref["ids"], ref["logits"], ref["ambiguous"]
    bad = []
    for t in range(ids_ref.shape[0]):
        if not amb[t]:
            if not np.array_equal(ids_gpu[t], ids_ref[t]):
                bad.append(t)
        else:
            kth = np.sort(lg[t])[::-1][k - 1]
            tol = 1e-5 * max(1.0, abs(kth))
            if len(set(ids_gpu[t].tolist())) != k or np.any(lg[t][ids_gpu[t]] < kth - tol):
                bad.append(t)
    return bad


def bf16_bits_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        (t.cpu().numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_layer(name: str, T: int):
    L = host_layer(name)
    x = synth.make_x(name, T)
    return x, OL.moe_layer(L, x)


def oracle_route_only(name: str, x: np.ndarray):
    L = host_layer(name)
    cfg = L["cfg"]
    ids, w, lg = OR.route(x, L["router_w"], L["router_bias"], cfg.k, cfg.score, cfg.bias_select_only)
    return {"ids": ids, "w": w, "logits": lg, "ambiguous": OR.ambiguous_tokens(lg, cfg.k)}


def gpu_hq_rows(dbg: dict, afmt: str, pairs) -> np.ndarray:
    """The GPU's re-quantized SwiGLU outputs of the given pairs, dequantized (FP64)."""
    from oracle import quant as OQ
    codes = dbg["hq_codes"].cpu().numpy()[pairs]
    if afmt == "nvfp4_4o6":
        return OQ.dequant_nvfp4_rows(codes, dbg["hq_scales"].cpu().numpy()[pairs],
                                     dbg["hq_scale"].cpu().numpy()[pairs])
    if afmt in ("mxfp4", "mxfp8"):
        return OQ.dequant_weights(afmt, codes, dbg["hq_scales"].cpu().numpy()[pairs], None)
    return OQ.dequant_fp8_token(codes, dbg["hq_scale"].cpu().numpy()[pairs])


def oracle_y_given_hq(name: str, x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray,
                      hq: np.ndarray) -> np.ndarray:
    """The oracle's layer output when the down projections take given quantized h rows
    hq [T, k, I] (FP64): y_t = sum_j w_tj * W2_e(tj) hq_tj + shared(x_t).

    For layers that re-quantize h, the GPU's FP32 h and the oracle's FP64 h differ in
    the last bits, which can move an element across a rounding boundary of the
    quantizer; the codes themselves are checked bit-exact against the oracle's
    quantizer fed the GPU's h, and this comparison then checks the rest of the layer."""
    L = host_layer(name)
    cfg = L["cfg"]
    T = x_bits.shape[0]
    y = np.zeros((T, cfg.H), dtype=np.float64)
    pos_of = {e: p for p, e in enumerate(L["expert_ids"])}
    for e in np.unique(ids):
        _, W2 = OL.expert_weights(L, "routed", pos_of[int(e)], cfg.wfmt)
        tt, jj = np.nonzero(ids == e)
        for t, j in zip(tt, jj):
            y[t] += w[t, j] * (W2 @ hq[t, j])
    if cfg.has_shared and T:
        from oracle.formats import bf16_to_f64
        W13, W2 = OL.expert_weights(L, "shared", 0, cfg.shared_wfmt)
        _, _, _, o = OL.mlp_rows(W13, W2, bf16_to_f64(x_bits), "bf16")
        y += o
    return y
