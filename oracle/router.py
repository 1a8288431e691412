"""FP64 router: logits, top-k selection and sigmoid or softmax combine weights (CPU oracle).

Test infrastructure (see oracle/__init__.py).

* "vLLM Day-0 support for Recursive's Flint", model architecture: 256 experts chosen
  by sigmoid top-6, plus one shared expert.
* "Inkling 2 Small on vLLM: Day-0 Support", architecture: sigmoid-routed MoE, 384
  routed experts, top-8; accuracy section: the router runs in FP32.
* "Day 0 support for Mistral Large 4 on vLLM", fusions: an FP32 router GEMM; ROCm
  implementation details (specialized decode): the fused decode runs a softmax top-4
  router.

Readings taken where the pages are silent: experts are selected by the k largest
logits (the sigmoid is monotone, so this is the same set as the k largest sigmoid
scores in exact arithmetic), ties go to the lower expert index, the selected sigmoid
scores are renormalised to sum to one, and an optional per-expert bias is added to
the logits before both selection and weighting. Softmax routing (the Mistral page gives
no more than its name): the same selection, with weights exp(l_j) / sum over the
selected of exp(l_j'), i.e. the softmax over all experts renormalised to the selection.
Selection-only bias (an option, not on the pages): the bias is added to the selection
keys only, and the weights use the bare logits.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64


def router_logits(x_bits: np.ndarray, router_w: np.ndarray, bias=None) -> np.ndarray:
    """logit[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]), in FP64."""
    x = bf16_to_f64(x_bits)
    lg = x @ np.asarray(router_w, dtype=np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)[None, :]
    return lg


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices [T, k] of the k largest logits per row, largest first, ties to lower index."""
    T, E = logits.shape
    out = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -logits[t]))   # primary key: -logit; secondary: index
        out[t] = order[:k]
    return out


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))),
                    np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))


def combine_weights(logits: np.ndarray, ids: np.ndarray, score: str = "sigmoid") -> np.ndarray:
    """w[t, j] = f(l[t, ids[t, j]]) / sum_j' f(l[t, ids[t, j']]), f = sigmoid, or exp
    for softmax (evaluated as exp(l - max over the selected), which cancels in the ratio)."""
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    if score == "sigmoid":
        s = sigmoid(sel)
    elif score == "softmax":
        s = np.exp(sel - sel.max(axis=1, keepdims=True))
    else:
        raise ValueError(score)
    return s / s.sum(axis=1, keepdims=True)


def ambiguous_tokens(logits: np.ndarray, k: int, rel: float = 1e-5) -> np.ndarray:
    """Tokens whose ranking among the top k+1 logits is decided by less than ``rel``.

    An FP32 router may legitimately order such near-equal logits differently from the
    FP64 oracle; tests accept either order for these tokens.
    """
    T, E = logits.shape
    amb = np.zeros(T, dtype=bool)
    n = min(k + 1, E)
    for t in range(T):
        srt = np.sort(logits[t])[::-1][:n]
        gaps = srt[:-1] - srt[1:]
        tol = rel * np.maximum(1.0, np.abs(srt[:-1]))
        amb[t] = bool(np.any(gaps < tol))
    return amb


def route(x_bits: np.ndarray, router_w: np.ndarray, bias, k: int, score: str = "sigmoid",
          bias_select_only: bool = False):
    """Returns (topk_ids [T, k] int32, topk_w [T, k] float64, keys [T, E] float64): the keys
    are the logits plus the bias, which select the experts; the weights take the keys, or
    the bare logits when bias_select_only."""
    keys = router_logits(x_bits, router_w, bias)
    ids = topk_select(keys, k)
    wl = router_logits(x_bits, router_w, None) if (bias is not None and bias_select_only) else keys
    return ids, combine_weights(wl, ids, score), keys
