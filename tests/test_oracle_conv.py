"""Pins for the fp64 oracle of the short causal convolution with boundary
state (the chunk's auxiliary local-convolution state: Pith review of
StateFlow, "What carries the argument", and Referee Report, major comment 1).

The oracle is checked against numpy's convolution routine on the extended
sequence, a closed form (a single tap shifts the input), the chunk-chaining
identity, the SiLU composition and central finite differences.
"""
import numpy as np
import pytest


def conv_inputs(rng, B, T, C, W, with_state=True):
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, W)) / W
    cin = rng.standard_normal((B, W - 1, C)) if with_state else None
    return x, w, cin


@pytest.mark.parametrize("B,T,C,W", [(1, 37, 5, 4), (2, 3, 4, 4), (1, 16, 3, 1), (2, 9, 2, 6)])
def test_matches_numpy_convolve(oracle_mod, B, T, C, W):
    rng = np.random.default_rng(11 + T + W)
    x, w, cin = conv_inputs(rng, B, T, C, W)
    y, cout = oracle_mod.shortconv_fwd(x, w, cin)
    for b in range(B):
        xe = np.concatenate([cin[b], x[b]], axis=0)
        for c in range(C):
            ref = np.convolve(xe[:, c], w[c], mode="valid")
            np.testing.assert_allclose(y[b, :, c], ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(cout[b], xe[xe.shape[0] - (W - 1):])


def test_single_tap_shifts_input(oracle_mod):
    """w = e_j: y_t = x_{t-j} (with the boundary state for t < j)."""
    rng = np.random.default_rng(3)
    B, T, C, W = 2, 12, 3, 4
    x, _, cin = conv_inputs(rng, B, T, C, W)
    for j in range(W):
        w = np.zeros((C, W))
        w[:, j] = 1.0
        y, _ = oracle_mod.shortconv_fwd(x, w, cin)
        xe = np.concatenate([cin, x], axis=1)
        np.testing.assert_array_equal(y, xe[:, W - 1 - j:W - 1 - j + T])


def test_zero_state_is_sequence_start(oracle_mod):
    rng = np.random.default_rng(4)
    x, w, _ = conv_inputs(rng, 1, 10, 2, 4, with_state=False)
    y0, _ = oracle_mod.shortconv_fwd(x, w, None)
    y1, _ = oracle_mod.shortconv_fwd(x, w, np.zeros((1, 3, 2)))
    np.testing.assert_array_equal(y0, y1)


@pytest.mark.parametrize("lengths", [[5, 1, 9, 2], [2, 2, 2], [1, 1, 1, 1, 1, 1]])
def test_chunk_chain_is_exact(oracle_mod, lengths):
    """Chunks chained through conv_out -> conv_in give the unchunked result
    bit for bit, forward and backward (including chunks shorter than W-1)."""
    rng = np.random.default_rng(5)
    B, C, W = 2, 3, 4
    T = sum(lengths)
    x, w, cin = conv_inputs(rng, B, T, C, W)
    dy = rng.standard_normal((B, T, C))
    dco = rng.standard_normal((B, W - 1, C))
    for act in (0, 1):
        y_ref, co_ref = oracle_mod.shortconv_fwd(x, w, cin, act)
        dx_ref, dw_ref, dci_ref = oracle_mod.shortconv_bwd(x, w, cin, dy, dco, act)
        bnd = np.cumsum([0] + lengths)
        state, ys, states = cin, [], [cin]
        for i in range(len(lengths)):
            sl = slice(bnd[i], bnd[i + 1])
            y, state = oracle_mod.shortconv_fwd(x[:, sl], w, state, act)
            ys.append(y)
            states.append(state)
        np.testing.assert_array_equal(np.concatenate(ys, axis=1), y_ref)
        np.testing.assert_array_equal(state, co_ref)
        g, dxs, dw = dco, [None] * len(lengths), np.zeros_like(w)
        for i in range(len(lengths) - 1, -1, -1):
            sl = slice(bnd[i], bnd[i + 1])
            dx, dwi, g = oracle_mod.shortconv_bwd(x[:, sl], w, states[i], dy[:, sl], g, act)
            dxs[i] = dx
            dw += dwi
        np.testing.assert_allclose(np.concatenate(dxs, axis=1), dx_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g, dci_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dw, dw_ref, rtol=1e-12, atol=1e-12)


def test_silu_is_applied_to_the_convolution(oracle_mod):
    rng = np.random.default_rng(6)
    x, w, cin = conv_inputs(rng, 2, 11, 3, 4)
    z, _ = oracle_mod.shortconv_fwd(x, w, cin, 0)
    y, _ = oracle_mod.shortconv_fwd(x, w, cin, 1)
    np.testing.assert_allclose(y, z / (1.0 + np.exp(-z)), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("act", [0, 1])
def test_backward_finite_differences(oracle_mod, act):
    """Directional derivatives of L = <dy, y> + <dco, conv_out> along random
    unit directions, for x, w and conv_in."""
    rng = np.random.default_rng(7 + act)
    B, T, C, W = 2, 6, 3, 4
    x, w, cin = conv_inputs(rng, B, T, C, W)
    dy = rng.standard_normal((B, T, C))
    dco = rng.standard_normal((B, W - 1, C))
    dx, dw, dci = oracle_mod.shortconv_bwd(x, w, cin, dy, dco, act)

    def loss(x_, w_, c_):
        y, co = oracle_mod.shortconv_fwd(x_, w_, c_, act)
        return float(np.sum(dy * y) + np.sum(dco * co))

    h = 1e-6
    for name, base, grad in (("x", x, dx), ("w", w, dw), ("cin", cin, dci)):
        u = rng.standard_normal(base.shape)
        u /= np.linalg.norm(u)
        args_p = {"x": x, "w": w, "cin": cin}
        args_m = dict(args_p)
        args_p[name] = base + h * u
        args_m[name] = base - h * u
        fd = (loss(args_p["x"], args_p["w"], args_p["cin"]) -
              loss(args_m["x"], args_m["w"], args_m["cin"])) / (2 * h)
        assert abs(fd - float(np.sum(grad * u))) < 1e-7 * max(1.0, abs(fd)), name
