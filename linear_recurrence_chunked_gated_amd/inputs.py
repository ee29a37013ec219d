"""Seeded synthetic inputs for one gated delta-rule chunk.

This module only draws random tensors; it holds none of the recurrence's
arithmetic and is shared by the tests (which hand the same tensors to the
device path and to the CPU oracle) and by the benchmark.

Recipe (the workloads the StateFlow page evaluates are Gated DeltaNet layers
on long sequences; no dataset is involved):
  q, k ~ N(0, 1), then L2-normalised per token in fp32;
  v ~ N(0, 1);
  beta = sigmoid(N(0, 1));
  alpha = exp(-decay * softplus(N(0, 1)))   (decay = 1, or 0.01 for the
          slow-decay variant in which the carried state matters; 10 and 0
          for the strong-decay and no-decay ends of the gate range);
  S_in ~ N(0, s_in_std) when requested, else absent (zeros);
  dO ~ N(0, 1), dS_out ~ N(0, ds_std) for backward runs.
Draw order: q, k, v, beta-logit, alpha-logit, S_in, dO, dS_out.
q, k, v and dO are then rounded to the run dtype; gates and states stay fp32.

On the CPU the draws come from numpy's PCG64; on a GPU device they come from
torch's device generator, so device-resident workloads never pass through
host memory.  Both are seeded; the two streams differ from each other.
"""
import numpy as np
import torch

_TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _softplus_np(x):
    return np.logaddexp(0.0, x)


def gdn_inputs(B, T, H, Dk, Dv, dtype="bf16", seed=0, s_in_std=None, grads=False,
               ds_std=0.1, decay=1.0, device="cpu"):
    """Return a dict of torch tensors on ``device``.

    Keys: q, k, v (run dtype), alpha, beta (fp32 [B,T,H]), S_in (fp32
    [B,H,Dv,Dk] or None); with grads=True also dO (run dtype) and dS_out
    (fp32 [B,H,Dv,Dk], or None when ds_std is None).
    """
    tdt = _TORCH_DTYPES[dtype]
    dev = torch.device(device)
    if dev.type == "cpu":
        rng = np.random.Generator(np.random.PCG64(seed))

        def normal(shape, std=1.0):
            return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))

        def post_gate(x, kind):
            if kind == "beta":
                return torch.from_numpy((1.0 / (1.0 + np.exp(-x.numpy().astype(np.float64))))
                                        .astype(np.float32))
            return torch.from_numpy(np.exp(-decay * _softplus_np(x.numpy().astype(np.float64)))
                                    .astype(np.float32))
    else:
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)

        def normal(shape, std=1.0):
            return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std

        def post_gate(x, kind):
            if kind == "beta":
                return torch.sigmoid(x)
            return torch.exp(-decay * torch.nn.functional.softplus(x))

    def unit_rows(x):
        n = torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x / n

    q = unit_rows(normal((B, T, H, Dk))).to(tdt)
    k = unit_rows(normal((B, T, H, Dk))).to(tdt)
    v = normal((B, T, H, Dv)).to(tdt)
    beta = post_gate(normal((B, T, H)), "beta").contiguous()
    alpha = post_gate(normal((B, T, H)), "alpha").contiguous()
    S_in = None
    if s_in_std is not None:
        S_in = normal((B, H, Dv, Dk), s_in_std).contiguous()
    out = {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
           "alpha": alpha.to(dev), "beta": beta.to(dev),
           "S_in": None if S_in is None else S_in.to(dev)}
    if grads:
        out["dO"] = normal((B, T, H, Dv)).to(tdt).contiguous()
        out["dS_out"] = None if ds_std is None else normal((B, H, Dv, Dk), ds_std).contiguous()
    for key in list(out):
        if out[key] is not None:
            out[key] = out[key].to(dev)
    return out


def conv_inputs(B, T, C, W, dtype="bf16", seed=0, state_std=1.0, grads=False, device="cpu"):
    """Seeded inputs for the short causal convolution of one chunk.

    Draw order: x ~ N(0, 1) [B,T,C]; w ~ N(0, 1) / W [C,W] (fp32);
    conv_in ~ N(0, state_std) [B,W-1,C] (None when state_std is None); with
    grads, dy ~ N(0, 1) [B,T,C] and dconv_out ~ N(0, 1) [B,W-1,C].  x, the
    states and dy are rounded to the run dtype; w stays fp32.  Same
    generators as gdn_inputs (numpy PCG64 on the CPU, torch on a device)."""
    tdt = _TORCH_DTYPES[dtype]
    dev = torch.device(device)
    if dev.type == "cpu":
        rng = np.random.Generator(np.random.PCG64(seed))

        def normal(shape, std=1.0):
            return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    else:
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)

        def normal(shape, std=1.0):
            return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std

    out = {"x": normal((B, T, C)).to(tdt).contiguous(),
           "w": (normal((C, W)) / W).contiguous(),
           "conv_in": None if state_std is None else
           normal((B, W - 1, C), state_std).to(tdt).contiguous()}
    if grads:
        out["dy"] = normal((B, T, C)).to(tdt).contiguous()
        out["dconv_out"] = normal((B, W - 1, C)).to(tdt).contiguous()
    return {k: (None if v is None else v.to(dev)) for k, v in out.items()}


def as_f64(t):
    """Exact float64 copy (numpy) of a tensor's stored values, for the oracle."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()


# The evaluation workloads, by shape.  Sizes are in tokens; "chunks" lists the
# pipeline-chunk lengths chained through the boundary state; "block" is the
# kernel block size.
WORKLOADS = {
    "fwd_f32_h2_t256_d64_4x64": dict(
        B=1, T=256, H=2, D=64, dtype="f32", chunks=[64] * 4, s_in_std=None, grads=False,
        seed=20260000),
    "fwd_bf16_h16_t8192_d128_8x1024": dict(
        B=1, T=8192, H=16, D=128, dtype="bf16", chunks=[1024] * 8, s_in_std=None, grads=False,
        seed=20260001),
    "fwd_bf16_h32_t65536_d128_sin": dict(
        B=1, T=65536, H=32, D=128, dtype="bf16", chunks=[65536], s_in_std=0.1, grads=False,
        seed=20260002),
    "fwdbwd_bf16_h16_t16384_d128": dict(
        B=1, T=16384, H=16, D=128, dtype="bf16", chunks=[16384], s_in_std=None, grads=True,
        seed=20260003),
    "fwdbwd_bf16_h16_t262144_d128_8skew": dict(
        B=1, T=262144, H=16, D=128, dtype="bf16", chunks="skew", s_in_std=None, grads=True,
        seed=20260004),
}
