"""The layer captured in a HIP graph: every replay must equal the eager result bit for
bit (the kernels use no memset and keep their counters consistent across replays)."""
import numpy as np
import pytest
import torch

import synth
from parity_util import device_layer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("flint_w4a16", 4), ("inkling_w4a4", 3), ("mistral_mxfp4_a8", 2),
                                    ("mistral_mxfp4_a4", 3)])
def test_graph_replays_match_eager(lib, name, T):
    say(f"[graph] {name} T={T}")
    dl = device_layer(name)
    ws = lib.Workspace(dl, T)
    x = torch.from_numpy(synth.make_x(name, T).view(np.int16)).cuda()
    ids, w, xq = lib.route(dl, x, ws)
    y = lib.expert_forward(dl, x, xq, ids, w, ws)
    torch.cuda.synchronize()
    y_eager = y.clone()
    ids_eager = ids.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.route(dl, x, ws, out=(ids, w, xq))
        lib.expert_forward(dl, x, xq, ids, w, ws, y=y)
    other = torch.from_numpy(synth.make_x(name, T + 1).view(np.int16)).cuda()
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_eager), rep
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep
        # eager work on the same workspace between replays (a different batch)
        i2, w2, q2 = lib.route(dl, other, lib.Workspace(dl, T + 1))
        torch.cuda.synchronize()


@pytest.mark.parametrize("name,T", [("flint_w4a16", 8), ("flint_w4a16", 2), ("flint_bf16", 8), ("tiny_bf16", 3)])
def test_graph_forward_replays_match_eager(lib, name, T):
    """moe_forward in a graph (routing fused into gate/up, token-mode down at these sizes):
    every replay equals the eager call, also after eager calls on other tokens on the same
    workspace in between, which equal the route + expert_forward path."""
    say(f"[graph] forward {name} T={T}")
    dl = device_layer(name)
    ws = lib.Workspace(dl, T)
    x = torch.from_numpy(synth.make_x(name, T).view(np.int16)).cuda()
    other = torch.from_numpy(synth.make_x(name, T + 1)[1:].copy().view(np.int16)).cuda()
    y, ids, w, xq = lib.forward(dl, x, ws)
    torch.cuda.synchronize()
    y_eager, ids_eager, w_eager = y.clone(), ids.clone(), w.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.forward(dl, x, ws, out=(y, ids, w, xq))
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_eager), rep
        assert torch.equal(w.view(torch.int32), w_eager.view(torch.int32)), rep
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep
        # an eager call on other tokens, same workspace, between replays
        y3, i3, w3, _ = lib.forward(dl, other, ws)
        i4, w4, q4 = lib.route(dl, other, ws)
        y4 = lib.expert_forward(dl, other, q4, i4, w4, ws)
        torch.cuda.synchronize()
        assert torch.equal(i3, i4), rep
        assert torch.equal(y3.view(torch.int16), y4.view(torch.int16)), rep
