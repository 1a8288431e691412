"""The layer captured in a HIP graph: every replay must equal the eager result bit for
bit (the kernels use no memset and keep their counters consistent across replays)."""
import numpy as np
import pytest
import torch

import synth
from parity_util import device_layer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("flint_w4a16", 4), ("inkling_w4a4", 3), ("mistral_mxfp4_a8", 2)])
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
