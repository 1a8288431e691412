"""One decode MoE layer, end to end, in FP64 (CPU oracle).

Test infrastructure (see oracle/__init__.py).

What the layer computes, as the pages describe it:
* router and sigmoid or softmax top-k (oracle/router.py);
* "vLLM Day-0 support for Recursive's Flint", optimization strategy: the expert GEMVs
  read only the selected experts' weights; routing and the expert combine sit next to
  them;
* "Inkling 2 Small on vLLM: Day-0 Support", MoE with fused activation quantization:
  the token is quantized before the gate/up projection and the SwiGLU output is
  quantized before the down projection (NVFP4 or MXFP8, matching the layer);
* "Day 0 support for Mistral Large 4 on vLLM", AMD section and ROCm implementation
  details: MXFP4 experts run with FP8 activations (a8w4) or, in the latency-specialized
  decode, with MXFP4 activations (a4w4); the Inkling page's MXFP8 expert layers quantize
  their activations to MXFP8. The MX activation formats follow the OCP MX v1.0 rule of
  oracle/quant.py (one E8M0 scale per 32 elements, floor(log2(block amax)) minus the
  element format's largest exponent), applied to each 32-block of a row;
* a shared expert is added to the routed mix with weight one (Flint and Mistral
  Large 4 architecture sections).

Plain definition, for token t with selected experts e_j and weights w_j:

    y_t = sum_j w_j * MLP_{e_j}(xhat_t) + [shared] * MLP_shared(x_t)
    MLP(v) = W2 @ Q_h(silu(Wg @ v) * (Wu @ v)),   silu(z) = z / (1 + exp(-z))

W* are the dequantized weights (FP64, exact). xhat and Q_h are identities except with
NVFP4 Four-Over-Six activations (both projections' inputs quantized per row), FP8
per-token activations (likewise), and MXFP4 / MXFP8 activations (both inputs quantized
per 32-block). The shared expert always sees the unquantized BF16
token and an unquantized SwiGLU output. "Soft-capped" SwiGLU is named on the Inkling
page without a constant; no cap is applied.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64
from .quant import (dequant_fp8_token, dequant_nvfp4_rows, dequant_weights,
                    quantize_fp8_token, quantize_mxfp4, quantize_mxfp8, quantize_nvfp4_4o6)
from .router import ambiguous_tokens, route

A_BF16, A_NVFP4_4O6, A_FP8_TOKEN = "bf16", "nvfp4_4o6", "fp8_token"
A_MXFP4, A_MXFP8 = "mxfp4", "mxfp8"


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def quantize_rows(afmt: str, v32: np.ndarray):
    """Quantize FP32 rows with activation format ``afmt``.

    Returns (dequantized FP64 rows, dict of the stored fields).
    """
    if afmt == A_NVFP4_4O6:
        codes, sb, g, choice = quantize_nvfp4_4o6(v32)
        return dequant_nvfp4_rows(codes, sb, g), {"codes": codes, "scales": sb, "g": g,
                                                 "choice": choice}
    if afmt == A_FP8_TOKEN:
        codes, s = quantize_fp8_token(v32)
        return dequant_fp8_token(codes, s), {"codes": codes, "s": s}
    if afmt in (A_MXFP4, A_MXFP8):
        codes, sc = (quantize_mxfp4 if afmt == A_MXFP4 else quantize_mxfp8)(v32)
        return dequant_weights(afmt, codes, sc, None), {"codes": codes, "scales": sc}
    return np.asarray(v32, dtype=np.float64), {}


def expert_weights(layer: dict, which: str, pos: int, fmt: str):
    """Dequantized (W13 [2I, H], W2 [H, I]) of stacked expert ``pos`` in ``which``."""
    if which == "routed":
        t13, t2 = layer["w13"], layer["w2"]
    else:
        t13, t2 = layer["sh13"], layer["sh2"]

    def tensor(t, rows_slice, gidx):
        codes = t["codes"][pos][rows_slice]
        scales = None if t["scales"] is None else t["scales"][pos][rows_slice]
        g = None if t["gscale"] is None else t["gscale"][pos][gidx]
        return dequant_weights(fmt, codes, scales, g)

    n13 = t13["codes"].shape[1]
    I = n13 // 2
    gate = tensor(t13, slice(0, I), 0)
    up = tensor(t13, slice(I, n13), 1)
    down = tensor(t2, slice(None), 0)
    return np.concatenate([gate, up], axis=0), down


def mlp_rows(W13: np.ndarray, W2: np.ndarray, X: np.ndarray, afmt_h: str):
    """SwiGLU MLP on rows X [n, H] (FP64). Returns (h [n, I], hq fields, hhat, o [n, H])."""
    I = W13.shape[0] // 2
    GU = X @ W13.T
    h = silu(GU[:, :I]) * GU[:, I:]
    if afmt_h == A_BF16:
        hhat, hq = h, {}
    else:
        hhat, hq = quantize_rows(afmt_h, h.astype(np.float32))
    return h, hq, hhat, hhat @ W2.T


def moe_layer(layer: dict, x_bits: np.ndarray) -> dict:
    """Run the layer on BF16 tokens x_bits [T, H] (uint16). FP64 throughout.

    Returns a dict with topk ids and weights, logits, the ambiguity mask, the
    quantized token fields, per-pair SwiGLU outputs h [T, k, I] (FP64), per-pair
    quantized h fields, the shared expert's h [T, I_shared] and y [T, H] (FP64).
    """
    cfg = layer["cfg"]
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0]
    ids, w, lg = route(x_bits, layer["router_w"], layer["router_bias"], cfg.k,
                       getattr(cfg, "score", "sigmoid"), getattr(cfg, "bias_select_only", False))
    x32 = bf16_to_f64(x_bits).astype(np.float32)          # exact
    x64 = x32.astype(np.float64)
    xhat, xq = quantize_rows(cfg.afmt, x32) if T else (x64, {})
    y = np.zeros((T, cfg.H), dtype=np.float64)
    h_pairs = np.zeros((T, cfg.k, cfg.I), dtype=np.float64)
    hq_pairs = [[None] * cfg.k for _ in range(T)]
    pos_of = {e: p for p, e in enumerate(layer["expert_ids"])}
    for e in np.unique(ids):
        W13, W2 = expert_weights(layer, "routed", pos_of[int(e)], cfg.wfmt)
        tt, jj = np.nonzero(ids == e)
        h, hq, _, o = mlp_rows(W13, W2, xhat[tt], cfg.afmt)
        for r, (t, j) in enumerate(zip(tt, jj)):
            h_pairs[t, j] = h[r]
            hq_pairs[t][j] = {key: val[r] for key, val in hq.items()}
            y[t] += w[t, j] * o[r]
    h_shared = None
    if cfg.has_shared and T:
        W13, W2 = expert_weights(layer, "shared", 0, cfg.shared_wfmt)
        h_shared, _, _, o = mlp_rows(W13, W2, x64, A_BF16)
        y += o
    return {"ids": ids, "w": w, "logits": lg, "ambiguous": ambiguous_tokens(lg, cfg.k),
            "xq": xq, "h": h_pairs, "hq": hq_pairs, "h_shared": h_shared, "y": y}

