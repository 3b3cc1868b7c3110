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


@pytest.mark.parametrize("name,n_ctx", [("c1", None), ("c2", None), ("c2", 777)])
def test_library_graph_matches_eager(name, n_ctx):
    """wenc_forward_graph: the forward recorded once by the library (both
    stream groups, every chunk) and replayed; every replay, with eager work
    and synchronisations between them, equals the eager forward bit for bit."""
    cfg, mel, _, _ = inputs(name)
    if n_ctx is not None:
        mel = np.ascontiguousarray(mel[:, :2 * n_ctx])
    say(f"library graph {name} n_ctx {n_ctx}")
    enc = encoder(name)
    m = dev(mel)
    eager = host(enc.forward(m, n_ctx=n_ctx))
    out = torch.empty_like(torch.from_numpy(eager)).to(m.device)
    for rep in range(4):
        out.fill_(float("nan"))
        enc.forward_graph(m, out, n_ctx=n_ctx)
        assert np.array_equal(host(out), eager), f"replay {rep}"
        _ = host(enc.forward(m, n_ctx=n_ctx))


def test_library_graph_rerecords_and_follows_reloads():
    """New buffers or sizes record a new graph; a graph replays with the
    weights the arena holds (wenc_load rewrites it in place); chunks of more
    windows than max_batch are recorded too; profiling refuses a graph."""
    from whisper_audio_encoder_amd import synth, wenc
    name = "c2"
    cfg, mel, params, blob = inputs(name)
    say("library graph: re-record, reload, chunks")
    enc = wenc.Encoder(cfg, blob, max_batch=3)  # batch 8 runs as 3 + 3 + 2 inside the graph
    try:
        m = dev(mel)
        eager = host(enc.forward(m))
        a = enc.forward_graph(m)
        assert np.array_equal(host(a), eager)
        five = host(enc.forward_graph(dev(mel[:5])))  # other buffers and batch: recorded anew
        assert np.array_equal(five, eager[:5])
        _, params2 = synth.make_inputs(cfg, seed=cfg.seed + 17)
        blob2 = synth.pack_blob(cfg, params2)
        wenc.wenc_load(enc.h, blob2)
        want = host(enc.forward(m))
        out = torch.empty_like(a)
        enc.forward_graph(m, out)
        enc.forward_graph(m, out)  # replay of the same recording
        assert np.array_equal(host(out), want) and not np.array_equal(want, eager)
        wenc.wenc_profile(enc.h, 1)
        with pytest.raises(wenc.WencError) as e:
            enc.forward_graph(m, out)
        assert e.value.code == wenc.WENC_ESTATE
        wenc.wenc_profile(enc.h, 0)
        wenc.wenc_profile_read(enc.h)
    finally:
        enc.close()
