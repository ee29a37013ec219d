"""A chunk past 2^31 elements per token tensor: B = 1, T = 1,100,001, H = 16,
d = 128, bf16 (2.25e9 elements, 4.5 GB per tensor), one call of the saving
forward and one of the saved backward, in the default plan (16 segments of
1,075 blocks per head, a ragged last block).  Element offsets pass 2^31 and
byte offsets 2^32 in every kernel.

The oracle cannot run 1.1M tokens per head within a test, so the chunk is cut
into independent windows by the method itself: at the two tokens R = 65,536
and R = T - 49,153 alpha is set to 1e-30, which scales the state carried into
R, and the state gradient carried back out of R, by 1e-30.  The window
[0, 65,536) is then a chunk of its own from the chunk's S_in with no exit
gradient, and [T - 49,153, T) one from a zero state with the chunk's dS_out;
each is checked against the oracle on two heads (0 and 15), the second
entirely above element 2^31.  dalpha at a cut token R depends on the state
before R and is left out; every other output of the windows is compared,
with the chunk's S_out and dS_in, at the bf16 bar (2e-2 per head).
Inputs are drawn on the device (as the benchmark draws them); only the
windows' heads are copied to the host.
"""
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from gdn_testutil import TOL, assert_close, inputs, oracle_args, f64, as_f64

pytestmark = pytest.mark.gpu

T, H, D = 1_100_001, 16, 128
CUT_A = 65_536
CUT_B = T - 49_153
HEADS = [0, 15]


def window(d, t0, t1, s_in, ds_out):
    """Tokens t0..t1-1 of heads HEADS as host tensors, with the given entry
    state and exit gradient (host tensors or None)."""
    out = {}
    for key in ("q", "k", "v", "dO"):
        out[key] = d[key][:, t0:t1, HEADS].cpu()
    for key in ("alpha", "beta"):
        out[key] = d[key][:, t0:t1, HEADS].cpu()
    out["S_in"] = s_in
    out["dS_out"] = ds_out
    return out


def test_chunk_past_2e31_elements(oracle_mod):
    assert T * H * D > 2 ** 31
    d = inputs(1, T, H, D, "bf16", seed=20261101, s_in_std=0.1, grads=True, device="cuda")
    d["alpha"][:, CUT_A] = 1e-30
    d["alpha"][:, CUT_B] = 1e-30
    o, S_out, saved = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"],
                                    saved=True)
    g = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, d["dO"],
                      d["dS_out"], saved=saved)
    torch.cuda.synchronize()
    del saved
    tol = TOL["bf16"]
    names = ("dq", "dk", "dv", "dalpha", "dbeta")
    for t0, t1, s_in, ds_out in ((0, CUT_A, d["S_in"][:, HEADS].cpu(), None),
                                 (CUT_B, T, None, d["dS_out"][:, HEADS].cpu())):
        w = window(d, t0, t1, s_in, ds_out)
        o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(w))
        tag = "[%d, %d)" % (t0, t1)
        assert_close("o " + tag, f64(o[:, t0:t1, HEADS]), o_ref, tol, head_axis=2)
        ref = oracle_mod.gdn_bwd(*oracle_args(w), as_f64(w["dO"]), as_f64(w["dS_out"]))
        for i, name in enumerate(names):
            got = f64(g[i][:, t0:t1, HEADS])
            want = ref[i]
            if name == "dalpha" and t0 > 0:
                got, want = got[:, 1:], want[:, 1:]  # the cut token itself
            assert_close(name + " " + tag, got, want, tol, head_axis=2)
        if t1 == T:
            assert_close("S_out", f64(S_out[:, HEADS]), S_ref, tol, head_axis=1)
        if t0 == 0:
            assert_close("dS_in", f64(g[5][:, HEADS]), ref[5], tol, head_axis=1)
