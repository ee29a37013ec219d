"""A chunk chain captured as a HIP graph (stream capture through torch) and
replayed: every replay, with eager work and synchronisations between the
replays, gives bit for bit the outputs of the same chain launched eagerly.
The library enqueues kernels only (no allocation, copy, memset or host
synchronisation inside a call), which is what capture needs.
"""
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from linear_recurrence_chunked_gated_amd import _lib
from gdn_testutil import inputs, to_dev

pytestmark = pytest.mark.gpu


def _chain_buffers(d, lengths, H, D):
    dev = d["q"].device
    n = len(lengths)
    shapes = [_lib.make_shape(1, t, H, D, D, d["q"].dtype) for t in lengths]
    return dict(
        o=torch.empty_like(d["v"]),
        states=[torch.zeros(1, H, D, D, device=dev)] + [torch.empty(1, H, D, D, device=dev)
                                                        for _ in range(n)],
        gst=[torch.empty(1, H, D, D, device=dev) for _ in range(n)],
        grads=[torch.empty_like(d[key]) for key in ("q", "k", "v", "alpha", "beta")],
        wsf=_lib.alloc_workspace(max(_lib.workspace_bytes(s) for s in shapes), dev),
        wsb=_lib.alloc_workspace(max(_lib.workspace_bytes(s, backward=True) for s in shapes), dev),
        saved=[_lib.alloc_workspace(_lib.saved_bytes(s), dev) for s in shapes],
    )


def _step(d, lengths, buf):
    """Saving forward then saved backward over the chunks, on the current stream."""
    bounds = [0]
    for t in lengths:
        bounds.append(bounds[-1] + t)
    q, k, v, al, be = d["q"], d["k"], d["v"], d["alpha"], d["beta"]
    for i in range(len(lengths)):
        sl = slice(bounds[i], bounds[i + 1])
        _lib.chunk_fwd(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl], buf["states"][i],
                       o=buf["o"][:, sl], S_out=buf["states"][i + 1], workspace=buf["wsf"],
                       saved=buf["saved"][i])
    G = d["dS_out"]
    for i in range(len(lengths) - 1, -1, -1):
        sl = slice(bounds[i], bounds[i + 1])
        _lib.chunk_bwd(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl], None, d["dO"][:, sl], G,
                       grads=tuple(g[:, sl] for g in buf["grads"]) + (buf["gst"][i],),
                       workspace=buf["wsb"], saved=buf["saved"][i])
        G = buf["gst"][i]


def _outputs(buf):
    return [buf["o"], buf["states"][-1], buf["gst"][0]] + list(buf["grads"])


@pytest.mark.parametrize("dtype,lengths", [
    ("bf16", [1024, 64, 1984, 960]),   # the 64-token chunk runs on the fp32 kernels
    ("f32", [1024, 64, 4608]),         # fp32 at d = 128: the gradient kernel's global tile areas, reused (288 blocks)
])
def test_graph_replays_equal_eager(dtype, lengths):
    H, D = 4, 128
    d = to_dev(inputs(1, sum(lengths), H, D, dtype, seed=31, grads=True, decay=0.01))
    buf = _chain_buffers(d, lengths, H, D)
    _step(d, lengths, buf)
    torch.cuda.synchronize()
    ref = [t.clone() for t in _outputs(buf)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(d, lengths, buf)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in _outputs(buf):
            t.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "S_out", "dS_in", "dq", "dk", "dv", "dalpha", "dbeta"),
                                   _outputs(buf), ref):
            assert torch.equal(got, want), "replay %d: %s differs from the eager run" % (rep, name)
