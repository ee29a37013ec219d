"""The autograd wrappers.  gated_delta_chunk: its gradients are exactly those
of the saving forward and saved backward called directly, chunks chained
through S_in = previous S_out differentiate as one sequence (against the fp64
oracle), and an output left out of the loss contributes a zero gradient.
short_conv: exactly the direct forward and backward calls, with and without a
boundary state, and for a window of one token."""
import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from gdn_testutil import TOL, assert_close, inputs, to_dev, oracle_args, f64, as_f64

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta")


def _leaves(dd, keys, s_in=True):
    out = {}
    for key in keys:
        t = dd[key]
        out[key] = None if t is None else t.detach().clone().requires_grad_(key != "S_in" or s_in)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,T", [("bf16", 128, 333), ("f32", 64, 200)])
def test_autograd_equals_direct_calls(dtype, D, T):
    d = inputs(2, T, 2, D, dtype, seed=4100 + T, s_in_std=0.1, grads=True, decay=0.05)
    dd = to_dev(d)
    x = _leaves(dd, ("q", "k", "v", "alpha", "beta", "S_in"))
    o, S_out = gdn.gated_delta_chunk(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S_in"],
                                     seg_blocks=2)
    loss = (o.float() * dd["dO"].float()).sum() + (S_out * dd["dS_out"]).sum()
    loss.backward()
    o2, S2, saved = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S_in"],
                                  seg_blocks=2, saved=True)
    ref = gdn.chunk_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None, dd["dO"],
                        dd["dS_out"], seg_blocks=2, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2) and torch.equal(S_out.detach(), S2)
    for key, r in zip(("q", "k", "v", "alpha", "beta", "S_in"), ref):
        assert torch.equal(x[key].grad, r), key


@pytest.mark.gpu
def test_autograd_chained_chunks_match_oracle(oracle_mod):
    """Three chunks of 512, 320 and 193 tokens, the second and third starting
    from the previous chunk's S_out, one loss over every o and the last
    S_out: the gradients of the whole sequence and of the first S_in."""
    lengths = (512, 320, 193)
    T = sum(lengths)
    d = inputs(1, T, 2, 128, "bf16", seed=4200, s_in_std=0.1, grads=True, decay=0.01)
    dd = to_dev(d)
    x = _leaves(dd, ("q", "k", "v", "alpha", "beta", "S_in"))
    S = x["S_in"]
    outs = []
    t0 = 0
    for n in lengths:
        sl = slice(t0, t0 + n)
        o, S = gdn.gated_delta_chunk(*(x[k][:, sl].contiguous()
                                       for k in ("q", "k", "v", "alpha", "beta")), S)
        outs.append(o)
        t0 += n
    o = torch.cat(outs, dim=1)
    loss = (o.float() * dd["dO"].float()).sum() + (S * dd["dS_out"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_fwd(*oracle_args(d))
    assert_close("o", f64(o), o_ref, TOL["bf16"], head_axis=2)
    assert_close("S_out", f64(S), S_ref, TOL["bf16"], head_axis=1)
    ref = oracle_mod.gdn_bwd(*oracle_args(d), as_f64(d["dO"]), as_f64(d["dS_out"]))
    for name, key, r in zip(NAMES + ("dS_in",), ("q", "k", "v", "alpha", "beta", "S_in"), ref):
        assert_close(name, f64(x[key].grad), r, TOL["bf16"], head_axis=1 if key == "S_in" else 2)


@pytest.mark.gpu
def test_autograd_unused_output_and_no_state():
    """S_out left out of the loss (its gradient arrives as zeros) and no S_in:
    the same gradients as the direct backward with dS_out = 0."""
    d = inputs(1, 200, 2, 64, "bf16", seed=4300, grads=True)
    dd = to_dev(d)
    x = _leaves(dd, ("q", "k", "v", "alpha", "beta"))
    o, _ = gdn.gated_delta_chunk(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    (o.float() * dd["dO"].float()).sum().backward()
    _, _, saved = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None,
                                saved=True)
    ref = gdn.chunk_bwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], None, dd["dO"],
                        torch.zeros_like(dd["dS_out"]), saved=saved)
    torch.cuda.synchronize()
    for key, r in zip(("q", "k", "v", "alpha", "beta"), ref):
        assert torch.equal(x[key].grad, r), key


def test_autograd_refuses_cpu_tensors():
    d = inputs(1, 64, 1, 64, "f32", seed=4400)
    with pytest.raises(ValueError):
        gdn.gated_delta_chunk(d["q"], d["k"], d["v"], d["alpha"], d["beta"])


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,W,act,state", [("bf16", 4, 1, True), ("f32", 4, 0, False),
                                               ("bf16", 1, 1, False)])
def test_short_conv_autograd_equals_direct_calls(dtype, W, act, state):
    from linear_recurrence_chunked_gated_amd.inputs import conv_inputs
    d = conv_inputs(2, 333, 136, W, dtype, seed=4500 + W, state_std=1.0 if state else None,
                    grads=True, device="cuda")
    x = d["x"].clone().requires_grad_(True)
    w = d["w"].clone().requires_grad_(True)
    ci = d["conv_in"].clone().requires_grad_(True) if state else None
    y, cout = gdn.short_conv(x, w, ci, act)
    loss = (y.float() * d["dy"].float()).sum()
    if W > 1:
        loss = loss + (cout.float() * d["dconv_out"].float()).sum()
    loss.backward()
    y2, c2 = gdn.shortconv_fwd(d["x"], d["w"], d["conv_in"] if state else None, act)
    ref = gdn.shortconv_bwd(d["x"], d["w"], d["conv_in"] if state else None, d["dy"],
                            d["dconv_out"] if W > 1 else None, act)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2)
    if W > 1:
        assert torch.equal(cout.detach(), c2)
    assert torch.equal(x.grad, ref[0]) and torch.equal(w.grad, ref[1])
    if state:
        assert torch.equal(ci.grad, ref[2])


def test_short_conv_refuses_cpu_tensors():
    from linear_recurrence_chunked_gated_amd.inputs import conv_inputs
    d = conv_inputs(1, 16, 64, 4, "f32", seed=4600)
    with pytest.raises(ValueError):
        gdn.short_conv(d["x"], d["w"], d["conv_in"])
