"""moe_forward_noalloc (the allocation-free variant of moe_forward, workspace in the
library's static per-GPU scratch) against moe_forward with a caller workspace: the same
ids, weights, quantized tokens and y, bit for bit, on two calls in a row, the second
with fewer tokens (so the scratch holds the first call's larger intermediates)."""
import numpy as np
import pytest
import torch

import synth
from parity_util import device_layer, say

pytestmark = pytest.mark.gpu

CASES = [
    ("flint_w4a16", (8, 3)),        # routing fused into gate/up, token-mode down
    ("inkling_w4a4", (8, 2)),       # quantized tokens and re-quantized h
    ("mistral_mxfp4_a8", (64, 33)), # grouped (MFMA) kernels, FP8 tokens
    ("tiny_bf16", (3, 1)),          # combine launch
]


def _same(a, b):
    if a is None:
        return b is None
    return np.array_equal(a.view(torch.uint8).cpu().numpy(), b.view(torch.uint8).cpu().numpy())


@pytest.mark.parametrize("name,Ts", CASES)
def test_noalloc_matches_forward(lib, name, Ts):
    dl = device_layer(name)
    ws = lib.Workspace(dl, max(Ts))
    for T in Ts:
        say(f"[noalloc] {name} T={T}")
        x = torch.from_numpy(synth.make_x(name, T).view(np.int16)).cuda()
        ref = lib.forward(dl, x, ws)
        got = lib.forward_noalloc(dl, x)
        torch.cuda.synchronize()
        for r, g, what in zip(ref, got, ("y", "ids", "w", "xq")):
            if what == "xq" and r is not None:
                pr, pg = lib.split_xq(dl, r, T), lib.split_xq(dl, g, T)
                for key in pr:
                    assert _same(pr[key], pg[key]), (what, key)
            else:
                assert _same(r, g), what


def test_noalloc_refuses_calls_past_its_scratch(lib):
    """Flint BF16 at 256 tokens needs about 21 MB of workspace: refused, nothing enqueued."""
    dl = device_layer("flint_bf16")
    T = 256
    need = lib.lib().moe_workspace_bytes(__import__("ctypes").byref(dl.struct), T)
    assert need > lib.noalloc_scratch_bytes()
    x = torch.from_numpy(synth.make_x("flint_bf16", T).view(np.int16)).cuda()
    with pytest.raises(lib.MoeError) as e:
        lib.forward_noalloc(dl, x)
    assert e.value.status == lib.MOE_EWORKSPACE
