"""Seeded synthetic MoE layers and activations.

This module only draws random numbers and stores them in the storage formats the
layer reads (raw E2M1 nibbles, E4M3 / E8M0 scale bytes, BF16 bit patterns, FP32).
It holds none of the layer's arithmetic: no dequantization, routing, quantizer or
matrix product. Rounding a random FP64 draw to BF16 or to an E4M3 scale byte is done
by PyTorch's dtype casts (round to nearest even). Both the CPU oracle and the GPU
path read the same arrays from here; neither imports the other.

Shapes follow the models the three pages describe:
  * "vLLM Day-0 support for Recursive's Flint", section on model architecture:
    hidden 2048, 256 experts with sigmoid top-6 plus one shared expert;
  * "Inkling 2 Small on vLLM: Day-0 Support", architecture table (Fig. 1): 384
    routed experts, top-8, no shared expert; NVFP4 and MXFP8 expert layers;
  * "Day 0 support for Mistral Large 4 on vLLM", highlights: hidden 6144, 128
    routed experts, top-4, one shared expert; AMD section: OCP MXFP4 experts.
The expert intermediate sizes are not on the pages; the values below are assumed.

Random streams: numpy PCG64 seeded with [0x4F36, config id, role, index]. Role 0 is
the router weight, 1 the router bias, 2 routed expert e (index e), 3 the shared
expert, 4 the activations (index T). One expert's tensors therefore do not depend on
how many other experts are drawn, so a test can rebuild any single expert.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

SEED_TAG = 0x4F36

# Storage formats of a weight tensor.
W_BF16, W_NVFP4, W_MXFP4, W_MXFP8 = "bf16", "nvfp4", "mxfp4", "mxfp8"
# Formats the routed experts' activations are quantized to before each projection.
A_BF16, A_NVFP4_4O6, A_FP8_TOKEN = "bf16", "nvfp4_4o6", "fp8_token"
A_MXFP4, A_MXFP8 = "mxfp4", "mxfp8"

# Expected rms of decode(E2M1 uniform over its 16 codes) * decode(E4M3 scale drawn
# log-uniform on [2^-8, 2^-2]): E[v^2] = 68.5/8 and E[S^2] = (2^-4 - 2^-16)/(12 ln 2).
# The FP32 global scale of each NVFP4 tensor is drawn around 0.02 / 0.2536 so that
# every tensor has an rms near 0.02, the spread of the BF16 configurations.
NVFP4_GSCALE_CENTER = 0.02 / 0.25364


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    cid: int
    H: int
    I: int
    E: int
    k: int
    has_shared: bool
    wfmt: str
    shared_wfmt: str
    afmt: str
    router_bias: bool = False
    x_outliers: bool = False
    batches: tuple = (1,)
    I_shared: Optional[int] = None
    score: str = "sigmoid"            # combine weights from "sigmoid" or "softmax" scores
    bias_select_only: bool = False    # the router bias enters the selection keys only

    @property
    def Ish(self) -> int:
        return self.I if self.I_shared is None else self.I_shared


CONFIGS: Dict[str, LayerConfig] = {
    # Tiny layer the oracle finishes in well under a second.
    "tiny_bf16": LayerConfig("tiny_bf16", 0, H=256, I=128, E=8, k=2, has_shared=True,
                             wfmt=W_BF16, shared_wfmt=W_BF16, afmt=A_BF16, batches=(1,)),
    # Flint-shaped, NVFP4 weights with BF16 activations (W4A16).
    "flint_w4a16": LayerConfig("flint_w4a16", 1, H=2048, I=768, E=256, k=6, has_shared=True,
                               wfmt=W_NVFP4, shared_wfmt=W_NVFP4, afmt=A_BF16,
                               batches=(1, 2, 4, 8)),
    # Flint-shaped, BF16 weights, router bias skews expert load.
    "flint_bf16": LayerConfig("flint_bf16", 2, H=2048, I=768, E=256, k=6, has_shared=True,
                              wfmt=W_BF16, shared_wfmt=W_BF16, afmt=A_BF16, router_bias=True,
                              batches=(1, 8, 64, 256)),
    # Inkling-2-Small-shaped, NVFP4 weights, activations quantized with Four Over Six.
    "inkling_w4a4": LayerConfig("inkling_w4a4", 3, H=4096, I=1536, E=384, k=8, has_shared=False,
                                wfmt=W_NVFP4, shared_wfmt=W_NVFP4, afmt=A_NVFP4_4O6,
                                x_outliers=True, batches=(1, 4, 8, 32)),
    # Inkling's MXFP8 expert layers with BF16 activations.
    "inkling_mxfp8": LayerConfig("inkling_mxfp8", 5, H=4096, I=1536, E=384, k=8, has_shared=False,
                                 wfmt=W_MXFP8, shared_wfmt=W_MXFP8, afmt=A_BF16,
                                 batches=(1, 8, 32)),
    # Mistral-Large-4-shaped, OCP MXFP4 routed experts, BF16 shared expert.
    "mistral_mxfp4": LayerConfig("mistral_mxfp4", 4, H=6144, I=2048, E=128, k=4, has_shared=True,
                                 wfmt=W_MXFP4, shared_wfmt=W_BF16, afmt=A_BF16,
                                 batches=(1, 8, 64)),
    # Same layer with FP8-E4M3 per-token activations on the routed experts (a8w4).
    "mistral_mxfp4_a8": LayerConfig("mistral_mxfp4_a8", 6, H=6144, I=2048, E=128, k=4,
                                    has_shared=True, wfmt=W_MXFP4, shared_wfmt=W_BF16,
                                    afmt=A_FP8_TOKEN, batches=(1, 8, 64)),
    # The Mistral-shaped layer's draws with OCP MXFP4 activations on the routed experts
    # (a4w4, the ROCm specialized decode of the Mistral Large 4 page).
    "mistral_mxfp4_a4": LayerConfig("mistral_mxfp4_a4", 4, H=6144, I=2048, E=128, k=4,
                                    has_shared=True, wfmt=W_MXFP4, shared_wfmt=W_BF16,
                                    afmt=A_MXFP4, batches=(1, 8, 64)),
    # Inkling's MXFP8 expert layers with their activations quantized to MXFP8 as well
    # (the Inkling page: fused activation quantization matching each layer's format).
    "inkling_mxfp8_a8": LayerConfig("inkling_mxfp8_a8", 5, H=4096, I=1536, E=384, k=8,
                                    has_shared=False, wfmt=W_MXFP8, shared_wfmt=W_MXFP8,
                                    afmt=A_MXFP8, batches=(1, 8, 32)),
    # Softmax top-k routing (the router of the Mistral Large 4 page's ROCm decode) on the
    # Mistral-shaped layer: the same draws as mistral_mxfp4.
    "mistral_mxfp4_softmax": LayerConfig("mistral_mxfp4_softmax", 4, H=6144, I=2048, E=128, k=4,
                                         has_shared=True, wfmt=W_MXFP4, shared_wfmt=W_BF16,
                                         afmt=A_BF16, score="softmax", batches=(1, 8, 64)),
    # Router bias used for expert selection only, on the bias-skewed Flint BF16 layer.
    "flint_bf16_selbias": LayerConfig("flint_bf16_selbias", 2, H=2048, I=768, E=256, k=6,
                                      has_shared=True, wfmt=W_BF16, shared_wfmt=W_BF16,
                                      afmt=A_BF16, router_bias=True, bias_select_only=True,
                                      batches=(1, 8, 64)),
    # Edge shapes: k = 1 over 5 experts (not a multiple of 64) at the smallest sizes; k = E
    # = 16 (the largest k, every expert selected); the largest E, 1024 (unfused top-k, 16
    # slots per lane).
    "edge_k1_e5": LayerConfig("edge_k1_e5", 8, H=256, I=128, E=5, k=1, has_shared=True,
                              wfmt=W_BF16, shared_wfmt=W_BF16, afmt=A_BF16, I_shared=256,
                              batches=(1, 7)),
    "edge_k16_e16": LayerConfig("edge_k16_e16", 9, H=512, I=256, E=16, k=16, has_shared=False,
                                wfmt=W_NVFP4, shared_wfmt=W_NVFP4, afmt=A_BF16, batches=(1, 3)),
    "edge_e1024": LayerConfig("edge_e1024", 10, H=512, I=256, E=1024, k=8, has_shared=False,
                              wfmt=W_MXFP4, shared_wfmt=W_MXFP4, afmt=A_BF16, batches=(1, 5)),
    # NVFP4 with rows longer than one batch of the GEMV walks (H = 1792: 7 batches per row;
    # I = 1280: 5), at a small expert count.
    "edge_nvfp4_batches": LayerConfig("edge_nvfp4_batches", 11, H=1792, I=1280, E=16, k=4,
                                      has_shared=True, wfmt=W_NVFP4, shared_wfmt=W_NVFP4,
                                      afmt=A_BF16, batches=(1, 4)),
    # Tiny layer with a router bias, softmax weights and selection-only bias.
    "tiny_softmax_selbias": LayerConfig("tiny_softmax_selbias", 7, H=256, I=128, E=8, k=2,
                                        has_shared=True, wfmt=W_BF16, shared_wfmt=W_BF16,
                                        afmt=A_BF16, router_bias=True, score="softmax",
                                        bias_select_only=True, batches=(1,)),
}


def rng_for(cid: int, role: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED_TAG, cid, role, index])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """FP64/FP32 draws -> BF16 bit patterns (uint16), via PyTorch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    """Positive draws <= 448 -> E4M3 bytes, via PyTorch's float8_e4m3fn RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _draw_tensor(rng: np.random.Generator, fmt: str, rows: int, K: int) -> dict:
    """One weight tensor [rows][K], K contiguous, in storage format ``fmt``."""
    if fmt == W_BF16:
        return {"codes": to_bf16_bits(rng.normal(0.0, 0.02, size=(rows, K))),
                "scales": None, "gscale": None}
    if fmt == W_NVFP4:
        codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)  # 2 uniform nibbles
        scales = to_e4m3_bits(np.exp2(rng.uniform(-8.0, -2.0, size=(rows, K // 16))))
        g = np.float32(NVFP4_GSCALE_CENTER * 2.0 ** rng.uniform(-0.25, 0.25))
        return {"codes": codes, "scales": scales, "gscale": g}
    if fmt == W_MXFP4:
        codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
        scales = (127 + rng.integers(-10, -1, size=(rows, K // 32))).astype(np.uint8)  # 2^-10..2^-2
        return {"codes": codes, "scales": scales, "gscale": None}
    if fmt == W_MXFP8:
        r = rng.integers(0, 254, size=(rows, K), dtype=np.int32)  # the 254 finite E4M3 bytes
        codes = (r + (r >= 0x7F)).astype(np.uint8)                # skip 0x7F, 0xFF (NaN)
        scales = (127 + rng.integers(-15, -10, size=(rows, K // 32))).astype(np.uint8)  # 2^-15..2^-11
        return {"codes": codes, "scales": scales, "gscale": None}
    raise ValueError(fmt)


def draw_expert(cfg: LayerConfig, role: int, index: int, fmt: str, I: int) -> dict:
    """gate/up stack W13 [2I][H] (gate rows first) and down W2 [H][I] of one expert."""
    rng = rng_for(cfg.cid, role, index)
    gate = _draw_tensor(rng, fmt, I, cfg.H)
    up = _draw_tensor(rng, fmt, I, cfg.H)
    down = _draw_tensor(rng, fmt, cfg.H, I)
    w13 = {"codes": np.concatenate([gate["codes"], up["codes"]], axis=0),
           "scales": None if gate["scales"] is None
           else np.concatenate([gate["scales"], up["scales"]], axis=0),
           "gscale": None if gate["gscale"] is None
           else np.array([gate["gscale"], up["gscale"]], dtype=np.float32)}
    w2 = {"codes": down["codes"], "scales": down["scales"],
          "gscale": None if down["gscale"] is None else np.array([down["gscale"]], np.float32)}
    return {"w13": w13, "w2": w2}


def _stack(parts: list, key: str) -> Optional[np.ndarray]:
    if not parts or parts[0][key] is None:
        return None
    return np.ascontiguousarray(np.stack([p[key] for p in parts], axis=0))


def make_layer(cfg: LayerConfig | str, experts: Optional[list] = None) -> dict:
    """Draw a whole layer (host numpy arrays).

    ``experts`` restricts the routed experts drawn to the given ids (the others are
    absent); None draws all E. Stacked tensors are [n][rows][...].
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    ids = list(range(cfg.E)) if experts is None else list(experts)
    rw = rng_for(cfg.cid, 0).normal(0.0, 0.05, size=(cfg.E, cfg.H)).astype(np.float32)
    bias = (rng_for(cfg.cid, 1).normal(0.0, 1.0, size=cfg.E).astype(np.float32)
            if cfg.router_bias else None)
    ex = [draw_expert(cfg, 2, e, cfg.wfmt, cfg.I) for e in ids]
    layer = {"cfg": cfg, "expert_ids": ids, "router_w": rw, "router_bias": bias,
             "w13": {k: _stack([p["w13"] for p in ex], k) for k in ("codes", "scales", "gscale")},
             "w2": {k: _stack([p["w2"] for p in ex], k) for k in ("codes", "scales", "gscale")},
             "sh13": None, "sh2": None}
    if cfg.has_shared:
        sh = draw_expert(cfg, 3, 0, cfg.shared_wfmt, cfg.Ish)
        layer["sh13"] = {k: None if v is None else v[None] for k, v in sh["w13"].items()}
        layer["sh2"] = {k: None if v is None else v[None] for k, v in sh["w2"].items()}
    return layer


def make_x(cfg: LayerConfig | str, T: int) -> np.ndarray:
    """Activations [T][H] as BF16 bits: N(0, 1); Inkling-shaped layers add 1 % outliers x20."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = rng_for(cfg.cid, 4, T)
    x = rng.normal(0.0, 1.0, size=(T, cfg.H))
    if cfg.x_outliers:
        x = np.where(rng.random(size=(T, cfg.H)) < 0.01, 20.0 * x, x)
    return to_bf16_bits(x)
