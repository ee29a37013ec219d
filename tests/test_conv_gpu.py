"""Short causal convolution with its chunk boundary state: the HIP kernels
through the C ABI against the fp64 oracle (Pith review of StateFlow, "What
carries the argument": a chunk's auxiliary local-convolution states).

Tolerance: max relative error per tensor <= 2e-2 for bf16, <= 1e-4 for fp32
(the same bar as the recurrence).  The weight gradient is a sum over all
tokens and is compared likewise.
"""
import numpy as np
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from linear_recurrence_chunked_gated_amd.inputs import conv_inputs, as_f64
from linear_recurrence_chunked_gated_amd.plan import chunk_lengths
from gdn_testutil import TOL, assert_close

pytestmark = pytest.mark.gpu


def run(d, act):
    dd = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    y, cout = gdn.shortconv_fwd(dd["x"], dd["w"], dd["conv_in"], act)
    dx, dw, dcin = gdn.shortconv_bwd(dd["x"], dd["w"], dd["conv_in"], dd["dy"], dd["dconv_out"],
                                     act)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else as_f64(t)
    return f(y), f(cout), f(dx), f(dw), f(dcin)


def oracle(oracle_mod, d, act):
    y, cout = oracle_mod.shortconv_fwd(as_f64(d["x"]), as_f64(d["w"]), as_f64(d["conv_in"]), act)
    dx, dw, dcin = oracle_mod.shortconv_bwd(as_f64(d["x"]), as_f64(d["w"]), as_f64(d["conv_in"]),
                                            as_f64(d["dy"]), as_f64(d["dconv_out"]), act)
    return y, cout, dx, dw, dcin


@pytest.mark.parametrize("B,T,C,W,dtype,act", [
    (1, 256, 64, 4, "f32", 0),
    (2, 100, 64, 4, "f32", 1),       # ragged against the token runs
    (2, 333, 136, 4, "bf16", 0),
    (1, 1000, 512, 4, "bf16", 1),
    (2, 3, 64, 4, "bf16", 1),        # chunk shorter than W-1 ... plus one
    (2, 2, 64, 4, "bf16", 0),        # chunk shorter than W-1
    (1, 1, 64, 4, "f32", 1),         # single token
    (1, 77, 72, 1, "bf16", 0),       # W = 1: no state
    (1, 300, 96, 8, "bf16", 1),      # widest supported window
    (1, 290, 96, 8, "bf16", 1),      # the last W-1 tokens span two token runs
    (2, 4096, 2048, 4, "bf16", 1),   # several runs per sequence
])
def test_matches_oracle(oracle_mod, B, T, C, W, dtype, act):
    d = conv_inputs(B, T, C, W, dtype, seed=4000 + T + C + W, grads=True)
    got = run(d, act)
    ref = oracle(oracle_mod, d, act)
    for name, g, r in zip(("y", "conv_out", "dx", "dw", "dconv_in"), got, ref):
        if W == 1 and name in ("conv_out", "dconv_in"):
            assert g is None
            continue
        assert_close(name, g, r, TOL[dtype])


def test_empty_chunk_passes_state():
    d = conv_inputs(2, 0, 64, 4, "bf16", seed=5, grads=True)
    dd = {k: v.cuda() for k, v in d.items()}
    y, cout = gdn.shortconv_fwd(dd["x"], dd["w"], dd["conv_in"])
    dx, dw, dcin = gdn.shortconv_bwd(dd["x"], dd["w"], dd["conv_in"], dd["dy"], dd["dconv_out"])
    torch.cuda.synchronize()
    assert torch.equal(cout, dd["conv_in"])
    assert torch.equal(dcin, dd["dconv_out"])
    assert torch.count_nonzero(dw) == 0


def test_chained_nonuniform_equals_unchunked(oracle_mod):
    """Eight skewed chunks chained through conv_out -> conv_in (forward) and
    dconv_in -> dconv_out (backward) against the unchunked oracle."""
    T, C, W = 8192, 256, 4
    lengths = chunk_lengths(T, 8, 0.5)
    d = conv_inputs(1, T, C, W, "bf16", seed=4100, state_std=None, grads=True)
    dd = {k: (None if v is None else v.cuda()) for k, v in d.items()}
    bnd = np.cumsum([0] + lengths)
    states, ys, state = [None], [], None
    for i in range(len(lengths)):
        sl = slice(int(bnd[i]), int(bnd[i + 1]))
        y, state = gdn.shortconv_fwd(dd["x"][:, sl], dd["w"], state, 1)
        ys.append(y)
        states.append(state)
    g, dxs, dw = None, [None] * len(lengths), torch.zeros_like(dd["w"])
    for i in range(len(lengths) - 1, -1, -1):
        sl = slice(int(bnd[i]), int(bnd[i + 1]))
        dx, dwi, g = gdn.shortconv_bwd(dd["x"][:, sl], dd["w"], states[i], dd["dy"][:, sl], g, 1)
        dxs[i] = dx
        dw += dwi
    torch.cuda.synchronize()
    y_ref, co_ref = oracle_mod.shortconv_fwd(as_f64(d["x"]), as_f64(d["w"]), None, 1)
    dx_ref, dw_ref, _ = oracle_mod.shortconv_bwd(as_f64(d["x"]), as_f64(d["w"]), None,
                                                 as_f64(d["dy"]), None, 1)
    assert_close("y", as_f64(torch.cat(ys, 1)), y_ref, TOL["bf16"])
    assert torch.equal(states[-1], dd["x"][:, T - (W - 1):])
    assert_close("dx", as_f64(torch.cat(dxs, 1)), dx_ref, TOL["bf16"])
    assert_close("dw", as_f64(dw), dw_ref, TOL["bf16"])


def test_full_size_sampled_channels(oracle_mod):
    """The largest chunk of the chained benchmark (62,720 tokens) over q, k
    and v of 16 heads at d = 128 (C = 6144), checked on a channel sample; the
    convolution is per channel, so the sample is exact."""
    T, C, W = 62720, 6144, 4
    d = conv_inputs(1, T, C, W, "bf16", seed=4200, grads=True)
    got = run(d, 1)
    cs = np.array([0, 1, 7, 1000, 2047, 2048, 4095, 6143])
    sub = {k: (None if v is None else (v[cs] if k == "w" else v[..., cs])) for k, v in d.items()}
    ref = oracle(oracle_mod, sub, 1)
    for name, g, r in zip(("y", "conv_out", "dx", "dw", "dconv_in"), got, ref):
        g = g[cs] if name == "dw" else g[..., cs]
        assert_close(name, g, r, TOL["bf16"])


def test_deterministic():
    d = conv_inputs(2, 3000, 512, 4, "bf16", seed=4300, grads=True)
    a = run(d, 1)
    b = run(d, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
