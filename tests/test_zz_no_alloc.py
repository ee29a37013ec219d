"""The no-allocation forward (sf_gdn_chunk_fwd_noalloc) against the
workspace forward (sf_gdn_chunk_fwd) it stands in for: the same kernels run
with the workspace in the library's static device array, so the outputs are
identical bit for bit.  Two calls in a row, the second with a smaller input,
so the second call runs on the array the first one left behind; and a shape
whose workspace exceeds the array is refused before anything runs."""
import ctypes

import pytest
import torch

import linear_recurrence_chunked_gated_amd as gdn
from linear_recurrence_chunked_gated_amd import _lib
from gdn_testutil import inputs, to_dev

pytestmark = pytest.mark.gpu


def _noalloc_c(d, o, S_out):
    """The entry point through the C ABI directly, on the current stream."""
    B, T, H, D = d["q"].shape
    shape = _lib.make_shape(B, T, H, D, D, d["q"].dtype)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return _lib.load().sf_gdn_chunk_fwd_noalloc(
        ctypes.byref(shape), p(d["q"]), p(d["k"]), p(d["v"]), p(d["alpha"]), p(d["beta"]),
        p(d["S_in"]), p(o), p(S_out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_noalloc_forward_equals_workspace_forward(dtype, D):
    cases = [(1, 8192, 4, 0.1), (2, 1000, 3, 0.1)]   # the second call smaller
    if dtype == "f32":
        cases = [(1, 2048, 2, 0.1), (1, 333, 2, None)]
    for i, (B, T, H, s_in) in enumerate(cases):
        d = to_dev(inputs(B, T, H, D, dtype, seed=5100 + i, s_in_std=s_in, decay=0.01))
        fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
        o1, S1 = gdn.chunk_fwd(*fa)
        o2 = torch.full_like(o1, float("nan"))
        S2 = torch.full_like(S1, float("nan"))
        assert _noalloc_c(d, o2, S2) == _lib.SF_OK, _lib.load().sf_last_error_message()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), (i, B, T, H)
        assert torch.equal(S1, S2), (i, B, T, H)


def test_noalloc_binding_and_size_limit():
    d = to_dev(inputs(1, 640, 2, 128, "bf16", seed=5200, s_in_std=0.1))
    fa = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S_in"])
    o1, S1 = gdn.chunk_fwd(*fa)
    o2, S2 = _lib.chunk_fwd_noalloc(*fa)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # 65,536 tokens x 16 heads needs about 176 MiB of workspace: refused
    big = _lib.make_shape(1, 65536, 16, 128, 128, torch.bfloat16)
    assert _lib.workspace_bytes(big) > 64 << 20
    L = _lib.load()
    G = 1 << 30
    vp = ctypes.c_void_p
    st = L.sf_gdn_chunk_fwd_noalloc(ctypes.byref(big), vp(G), vp(2 * G), vp(3 * G), vp(4 * G),
                                    vp(5 * G), None, vp(6 * G), vp(7 * G), None)
    assert st == _lib.SF_ERR_WORKSPACE
    assert "scratch" in L.sf_last_error_message().decode()
