"""NaN propagation and stream handling of the chunk calls.

The library does not check inputs for finiteness (that would cost a pass over
HBM); a NaN in one (batch, head) sequence must reach that sequence's outputs
and leave every other sequence's outputs bit for bit as without it, since
the sequences are independent.  Buffers the binding allocates for a call on a
stream other than the current one must stay reserved until the kernels on
that stream are done.
"""
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from gdn_testutil import inputs, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS_in")


def _heads_equal(x, y, axis, skip):
    for h in range(x.shape[axis]):
        if h == skip:
            continue
        assert torch.equal(x.select(axis, h), y.select(axis, h)), h


@pytest.mark.parametrize("where", ["v", "k", "alpha", "beta", "S_in"])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32"), (128, "f32")])
def test_forward_nan_stays_in_its_sequence(where, D, dtype):
    d = to_dev(inputs(2, 700, 3, D, dtype, seed=61, s_in_std=0.1, decay=0.05))
    fa = [d[k] for k in ("q", "k", "v", "alpha", "beta", "S_in")]
    o1, S1 = gdn.chunk_fwd(*fa)
    bad = {k: t.clone() for k, t in zip(("q", "k", "v", "alpha", "beta", "S_in"), fa)}
    b, t, h = 1, 130, 2
    if where == "S_in":
        bad["S_in"][b, h, 5, 7] = float("nan")
    elif where in ("alpha", "beta"):
        bad[where][b, t, h] = float("nan")
    else:
        bad[where][b, t, h, 3] = float("nan")
    o2, S2 = gdn.chunk_fwd(*bad.values())
    torch.cuda.synchronize()
    assert torch.isnan(o2[b, :, h]).any() and torch.isnan(S2[b, h]).any()
    assert torch.equal(o1[0], o2[0]) and torch.equal(S1[0], S2[0])  # the other batch row
    _heads_equal(o1[b], o2[b], 1, h)
    _heads_equal(S1[b], S2[b], 0, h)


@pytest.mark.parametrize("saved", [False, True])
def test_backward_nan_stays_in_its_sequence(saved):
    d = to_dev(inputs(1, 1000, 3, 128, "bf16", seed=62, s_in_std=0.1, grads=True, decay=0.05))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    sv = gdn.chunk_fwd(*fa, saved=True)[2] if saved else None
    dO2 = d["dO"].clone()
    dO2[0, 500, 1, 9] = float("nan")
    if saved:
        g1 = gdn.chunk_bwd(*fa[:5], None, d["dO"], d["dS_out"], saved=sv)
        g2 = gdn.chunk_bwd(*fa[:5], None, dO2, d["dS_out"], saved=sv)
    else:
        g1 = gdn.chunk_bwd(*fa, d["dO"], d["dS_out"])
        g2 = gdn.chunk_bwd(*fa, dO2, d["dS_out"])
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, g1, g2):
        axis = 1 if name == "dS_in" else 2
        assert torch.isnan(y.select(axis, 1)).any(), name
        _heads_equal(x, y, axis, 1)


def test_backward_nan_stays_in_its_sequence_fp32_d128():
    """fp32 at d = 128, whose gradient kernel keeps its input tiles in a
    global area per workgroup and strides over the blocks (B * H * nblk =
    384 blocks against 256 workgroups, so areas are reused): a NaN in one
    sequence's dO reaches that sequence's gradients only, and the other
    sequences' gradients are bit for bit those of the clean run."""
    d = to_dev(inputs(2, 4000, 3, 128, "f32", seed=64, s_in_std=0.1, grads=True, decay=0.05))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    dO2 = d["dO"].clone()
    b, t, h = 0, 2500, 1
    dO2[b, t, h, 9] = float("nan")
    g1 = gdn.chunk_bwd(*fa, d["dO"], d["dS_out"])
    g2 = gdn.chunk_bwd(*fa, dO2, d["dS_out"])
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, g1, g2):
        axis = 0 if name == "dS_in" else 1  # batch-major views: [B, H, ...] or [B, T, H, ...]
        assert torch.isnan(y[b].select(axis, h)).any(), name
        assert torch.equal(x[1 - b], y[1 - b]), name  # the other batch row
        _heads_equal(x[b], y[b], axis, h)


def test_chains_on_a_side_stream_equal_current_stream():
    """Chunk chains launched on a non-current stream, with the binding
    allocating workspaces and outputs itself, give the current-stream results
    bit for bit while other work on the current stream allocates and writes
    memory meanwhile."""
    lengths = [1000, 64, 1936]
    d = to_dev(inputs(1, sum(lengths), 2, 128, "bf16", seed=63, s_in_std=0.1, grads=True,
                      decay=0.01))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    o1, st1, sv1 = gdn.chain_fwd(*fa, lengths, save=True)
    g1 = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, None, saved=sv1)
    g1r = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, st1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o2, st2, sv2 = gdn.chain_fwd(*fa, lengths, save=True, stream=side)
    g2 = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, None, saved=sv2, stream=side)
    g2r = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, st2, stream=side)
    for _ in range(8):  # current-stream work that reuses freed memory if it may
        torch.empty(96 << 20, dtype=torch.uint8, device="cuda").fill_(0x7f)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for a, b in zip(st1, st2):
        assert torch.equal(a, b)
    for name, x, y, xr, yr in zip(NAMES, g1, g2, g1r, g2r):
        assert torch.equal(x, y), name
        assert torch.equal(xr, yr), name
