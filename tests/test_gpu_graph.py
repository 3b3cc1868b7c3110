"""wenc_forward captured into a hipGraph (torch.cuda.CUDAGraph) and replayed.

The forward enqueues kernels only (no memset, no host synchronisation), so
it can be captured.  Each replay is checked against the eager result, with
the program's own eager work and synchronisations between replays.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev, host, say
from tests.test_gpu_encoder import encoder, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_ctx", [("c1", None), ("c2", None), ("c2", 500)])
def test_graph_replay_matches_eager(name, n_ctx):
    cfg, mel, _, _ = inputs(name)
    if n_ctx is not None:
        mel = np.ascontiguousarray(mel[:, :2 * n_ctx])
    say(f"graph replay {name} n_ctx {n_ctx}")
    enc = encoder(name)
    m = dev(mel)
    eager = host(enc.forward(m, n_ctx=n_ctx))
    out = torch.empty_like(torch.from_numpy(eager)).to(m.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enc.forward(m, out, n_ctx=n_ctx)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enc.forward(m, out, n_ctx=n_ctx)
    for rep in range(4):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = host(out)
        assert np.array_equal(got, eager), f"replay {rep}"
        _ = host(enc.forward(m, n_ctx=n_ctx))  # an eager forward in between
    del g
