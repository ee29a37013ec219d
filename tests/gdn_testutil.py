"""Shared helpers for the device-vs-oracle tests (not a test module)."""
import numpy as np
import torch

from linear_recurrence_chunked_gated_amd.inputs import gdn_inputs, as_f64

TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel_err(x, ref, head_axis=None):
    """max |x - ref| / max |ref|; with head_axis, the worst head's value."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise AssertionError("shape %s vs %s" % (x.shape, ref.shape))
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    if head_axis is None:
        den = np.abs(ref).max()
        return float(np.abs(x - ref).max() / den) if den > 0 else float(np.abs(x).max())
    xs = np.moveaxis(x, head_axis, 0)
    rs = np.moveaxis(ref, head_axis, 0)
    worst = 0.0
    for a, b in zip(xs, rs):
        den = np.abs(b).max()
        e = np.abs(a - b).max() / den if den > 0 else np.abs(a).max()
        worst = max(worst, float(e))
    return worst


def frob_err(x, ref):
    """||x - ref||_F / ||ref||_F (reported beside the max-relative bar)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def assert_close(name, x, ref, tol, head_axis=None):
    e = rel_err(x, ref, head_axis)
    assert e <= tol, "%s: max relative error %.3e > %.1e (relative Frobenius error %.3e)" % (
        name, e, tol, frob_err(x, ref))
    return e


def inputs(B, T, H, D, dtype, seed, s_in_std=None, grads=False, decay=1.0, ds_std=0.1,
           device="cpu"):
    return gdn_inputs(B, T, H, D, D, dtype=dtype, seed=seed, s_in_std=s_in_std, grads=grads,
                      decay=decay, ds_std=ds_std, device=device)


def to_dev(d, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in d.items()}


def oracle_args(d):
    return [as_f64(d[k]) for k in ("q", "k", "v", "alpha", "beta")] + [as_f64(d.get("S_in"))]


def head_slice(d, hs):
    """Inputs restricted to heads hs (copies), for sampled oracle checks."""
    out = {}
    for key, t in d.items():
        if t is None:
            out[key] = None
        elif key in ("S_in", "dS_out"):
            out[key] = t[:, hs].contiguous()
        else:
            out[key] = t[:, :, hs].contiguous()
    return out


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()
