"""Split-and-overlap of consecutive chunks (the two launch groups of a chunk
call, sf_gdn_chunk_fwd_split and sf_gdn_chunk_bwd_saved_split): BEGIN then
END equals one whole call bit for bit, and the overlapped chunk chains (the
next chunk's state-independent launches on a second stream) equal the plain
chains bit for bit and the unchunked fp64 oracle within the bf16 bar, per
head."""
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from linear_recurrence_chunked_gated_amd import _lib
from linear_recurrence_chunked_gated_amd.plan import chunk_lengths
from gdn_testutil import TOL, assert_close, inputs, to_dev, oracle_args, f64, as_f64

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 256, 2, 64, "f32", 1),     # fp32, one block per segment
    (1, 1000, 3, 128, "bf16", 0),  # ragged, several segments
    (1, 640, 2, 128, "bf16", 100),  # one segment
    (1, 1, 2, 128, "bf16", 0),     # single token
    (2, 2048, 2, 128, "bf16", 5),
    (1, 0, 2, 64, "bf16", 0),      # empty chunk
]


@pytest.mark.parametrize("B,T,H,D,dtype,seg", SHAPES)
@pytest.mark.parametrize("save", [False, True])
def test_split_forward_equals_whole(B, T, H, D, dtype, seg, save):
    d = to_dev(inputs(B, T, H, D, dtype, seed=4000 + T, s_in_std=0.1, decay=0.01))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    shape = _lib.make_shape(B, T, H, D, D, d["q"].dtype, seg)
    ws = _lib.alloc_workspace(max(_lib.workspace_bytes(shape), 256), d["q"].device)
    n_sv = _lib.saved_bytes(shape)
    sv1 = _lib.alloc_workspace(max(n_sv, 256), d["q"].device) if save else None
    sv2 = _lib.alloc_workspace(max(n_sv, 256), d["q"].device) if save else None
    r1 = gdn.chunk_fwd(*fa, seg_blocks=seg, saved=sv1)
    o2 = torch.empty_like(r1[0])
    S2 = torch.empty_like(r1[1])
    gdn.chunk_fwd(*fa, o=o2, S_out=S2, seg_blocks=seg, workspace=ws, saved=sv2,
                  phase=_lib.PHASE_BEGIN)
    gdn.chunk_fwd(*fa, o=o2, S_out=S2, seg_blocks=seg, workspace=ws, saved=sv2,
                  phase=_lib.PHASE_END)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], o2) and torch.equal(r1[1], S2)
    if save:
        assert torch.equal(sv1[:n_sv], sv2[:n_sv])


@pytest.mark.parametrize("B,T,H,D,dtype,seg", SHAPES)
def test_split_saved_backward_equals_whole(B, T, H, D, dtype, seg):
    d = to_dev(inputs(B, T, H, D, dtype, seed=4100 + T, s_in_std=0.1, grads=True, decay=0.01))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    _, _, saved = gdn.chunk_fwd(*fa, seg_blocks=seg, saved=True)
    g1 = gdn.chunk_bwd(*fa[:5], None, d["dO"], d["dS_out"], seg_blocks=seg, saved=saved)
    shape = _lib.make_shape(B, T, H, D, D, d["q"].dtype, seg)
    ws = _lib.alloc_workspace(max(_lib.workspace_bytes(shape, backward=True), 256),
                              d["q"].device)
    g2 = tuple(torch.empty_like(x) for x in g1)
    for ph in (_lib.PHASE_BEGIN, _lib.PHASE_END):
        gdn.chunk_bwd(*fa[:5], None, d["dO"], d["dS_out"], grads=g2, seg_blocks=seg,
                      workspace=ws, saved=saved, phase=ph)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_in"), g1, g2):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("lengths,H", [(chunk_lengths(16384, 8, 0.5), 4),
                                       ([1000, 64, 1936], 2),   # ragged, odd count
                                       ([1000], 2)])
def test_overlapped_chains_equal_plain(oracle_mod, lengths, H):
    T, n = sum(lengths), len(lengths)
    d = to_dev(inputs(1, T, H, 128, "bf16", seed=4200 + n, s_in_std=0.1, grads=True,
                      decay=0.01))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    o1, st1, sv1 = gdn.chain_fwd(*fa, lengths, save=True)
    o2, st2, sv2 = gdn.chain_fwd(*fa, lengths, save=True, overlap=True)
    o3, st3 = gdn.chain_fwd(*fa, lengths, overlap=True)
    g1 = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, None, saved=sv1)
    g2 = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, None, saved=sv2, overlap=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    for a, b, c in zip(st1, st2, st3):
        assert torch.equal(a, b) and torch.equal(a, c)
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_in"), g1, g2):
        assert torch.equal(x, y), name
    # the overlapped chains against the unchunked oracle (chunking is exact in
    # real arithmetic: Eqs. 5 and 7)
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    for o in (o2, o3):
        assert_close("o", f64(o), o_ref, TOL["bf16"], head_axis=2)
    for st in (st2, st3):
        assert_close("S_out", f64(st[-1]), S_ref, TOL["bf16"], head_axis=1)
    g_ref = oracle_mod.gdn_bwd(*oracle_args(d), as_f64(d["dO"]), as_f64(d["dS_out"]))
    for name, x, r, ax in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_in"), g2, g_ref,
                              (2, 2, 2, 2, 2, 1)):
        assert_close(name, f64(x), r, TOL["bf16"], head_axis=ax)


@pytest.mark.parametrize("f", [0.5, 0.7])
def test_split_fraction_chains(oracle_mod, f):
    """Every chunk cut at fraction f into two parts (the page's split for
    overlap), overlapped on two streams: bit for bit the same split run on
    one stream, and the unchunked oracle within the bf16 bar, per head."""
    lengths = chunk_lengths(16384, 8, 0.5)
    d = to_dev(inputs(1, sum(lengths), 4, 128, "bf16", seed=4300, s_in_std=0.1, grads=True,
                      decay=0.01))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    o1, st1, sv1 = gdn.chain_fwd(*fa, lengths, save=True, split=f)
    g1 = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, None, saved=sv1, split=f)
    o2, st2, sv2 = gdn.chain_fwd(*fa, lengths, save=True, overlap=True, split=f)
    g2 = gdn.chain_bwd(*fa[:5], d["dO"], d["dS_out"], lengths, None, saved=sv2, overlap=True,
                       split=f)
    torch.cuda.synchronize()
    assert len(sv1) == 2 * len(lengths)
    assert torch.equal(o1, o2) and torch.equal(st1[-1], st2[-1])
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_in"), g1, g2):
        assert torch.equal(x, y), name
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o2), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(st2[-1]), S_ref, TOL["bf16"], head_axis=1)
    g_ref = oracle_mod.gdn_bwd(*oracle_args(d), as_f64(d["dO"]), as_f64(d["dS_out"]))
    for name, x, r, ax in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS_in"), g2, g_ref,
                              (2, 2, 2, 2, 2, 1)):
        assert_close(name, f64(x), r, TOL["bf16"], head_axis=ax)
