"""Host-side checks that need no GPU: the C ABI library loads and exports
every declared symbol, arguments are validated before anything is enqueued,
and the chunk planner matches the oracle's search."""
import ctypes
import os
import re

import pytest

from linear_recurrence_chunked_gated_amd import _lib
from linear_recurrence_chunked_gated_amd.plan import chunk_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sf_gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(sf_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_chunk_calls():
    names = declared_functions()
    for n in ("sf_gdn_chunk_fwd", "sf_gdn_chunk_bwd", "sf_gdn_chunk_fwd_workspace_size",
              "sf_gdn_chunk_bwd_workspace_size", "sf_status_string", "sf_last_error_message"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding describes each declared function
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def _shape(B=1, T=128, H=2, D=128, dtype=1, seg=0):
    return _lib.Shape(B, T, H, D, D, dtype, seg)


G = 1 << 30  # fake, never dereferenced: validation fails before any launch


def _fwd(shape, q=1 * G, k=2 * G, v=3 * G, a=4 * G, b=5 * G, s_in=None,
         o=6 * G, s_out=7 * G, ws=None, wsn=0):
    L = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.sf_gdn_chunk_fwd(ctypes.byref(shape) if shape is not None else None,
                              vp(q), vp(k), vp(v), vp(a), vp(b), vp(s_in), vp(o), vp(s_out),
                              vp(ws), ctypes.c_size_t(wsn), None)


def test_status_strings():
    assert _lib.status_string(0) == "SF_OK"
    assert _lib.status_string(3) == "SF_ERR_WORKSPACE"


@pytest.mark.parametrize("shape,code", [
    (_shape(B=0), _lib.SF_ERR_INVALID_ARG),
    (_shape(T=-1), _lib.SF_ERR_INVALID_ARG),
    (_shape(D=96), _lib.SF_ERR_UNSUPPORTED),
    (_shape(dtype=7), _lib.SF_ERR_INVALID_ARG),
    (_shape(seg=-2), _lib.SF_ERR_INVALID_ARG),
])
def test_rejects_bad_shapes(shape, code):
    assert _fwd(shape) == code
    assert _lib.load().sf_last_error_message()


def test_rejects_null_shape_and_missing_pointers():
    assert _fwd(None) == _lib.SF_ERR_INVALID_ARG
    assert _fwd(_shape(), q=None) == _lib.SF_ERR_INVALID_ARG
    assert _fwd(_shape(), o=None) == _lib.SF_ERR_INVALID_ARG


def test_rejects_misaligned_and_overlapping():
    assert _fwd(_shape(), q=G + 2) == _lib.SF_ERR_INVALID_ARG
    # o overlapping q
    assert _fwd(_shape(), o=G + 64) == _lib.SF_ERR_INVALID_ARG
    # S_out overlapping o
    assert _fwd(_shape(), s_out=6 * G + 256) == _lib.SF_ERR_INVALID_ARG
    msg = _lib.load().sf_last_error_message().decode()
    assert "overlaps" in msg


def test_rejects_small_workspace():
    shape = _shape(T=8192, H=2)
    need = _lib.workspace_bytes(shape)
    assert need > 0
    assert _fwd(shape, ws=16 * G, wsn=need - 1) == _lib.SF_ERR_WORKSPACE
    assert _fwd(shape, ws=None, wsn=0) == _lib.SF_ERR_WORKSPACE
    assert _fwd(shape, ws=16 * G + 16, wsn=need) == _lib.SF_ERR_INVALID_ARG  # not 256-aligned


def _fwd_save(shape, saved=20 * G, svn=None, ws=24 * G, wsn=None):
    L = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    svn = _lib.saved_bytes(shape) if svn is None else svn
    wsn = _lib.workspace_bytes(shape) if wsn is None else wsn
    return L.sf_gdn_chunk_fwd_save(ctypes.byref(shape), vp(1 * G), vp(2 * G), vp(3 * G),
                                   vp(4 * G), vp(5 * G), None, vp(6 * G), vp(7 * G), vp(saved),
                                   ctypes.c_size_t(svn), vp(ws), ctypes.c_size_t(wsn), None)


def _bwd_saved(shape, saved=20 * G, svn=None, ws=24 * G, wsn=None, dq=8 * G):
    L = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    svn = _lib.saved_bytes(shape) if svn is None else svn
    wsn = _lib.workspace_bytes(shape, backward=True) if wsn is None else wsn
    return L.sf_gdn_chunk_bwd_saved(ctypes.byref(shape), vp(1 * G), vp(2 * G), vp(3 * G),
                                    vp(4 * G), vp(5 * G), vp(saved), ctypes.c_size_t(svn),
                                    vp(6 * G), None, vp(dq), vp(9 * G), vp(10 * G), vp(11 * G),
                                    vp(12 * G), None, vp(ws), ctypes.c_size_t(wsn), None)


def test_saved_buffer_validation():
    shape = _shape(T=8192, H=2)
    need = _lib.saved_bytes(shape)
    # at least the per-block entry states and Tp, Tpp, in bf16, of 2 heads
    nblk = 8192 // 64
    assert need >= 2 * nblk * (128 * 128 + 2 * 64 * 64) * 2
    for call in (_fwd_save, _bwd_saved):
        assert call(shape, svn=need - 1) == _lib.SF_ERR_INVALID_ARG
        assert "saved" in _lib.load().sf_last_error_message().decode()
        assert call(shape, saved=None, svn=0) == _lib.SF_ERR_INVALID_ARG
        assert call(shape, saved=20 * G + 64) == _lib.SF_ERR_INVALID_ARG  # not 256-aligned
    # the saving forward writes it: it must not overlap an input
    assert _fwd_save(shape, saved=3 * G + 256) == _lib.SF_ERR_INVALID_ARG
    assert _bwd_saved(shape, dq=20 * G + 4096) == _lib.SF_ERR_INVALID_ARG  # dq overlaps saved
    # an empty chunk needs no saved buffer
    assert _lib.saved_bytes(_shape(T=0)) == 0


def test_workspace_sizes():
    # one segment needs no forward workspace
    assert _lib.workspace_bytes(_shape(T=64, H=1, seg=0)) >= 0
    s = _shape(B=1, T=65536, H=16, D=128)
    f = _lib.workspace_bytes(s)
    b = _lib.workspace_bytes(s, backward=True)
    assert b > f > 0
    # explicit segment length changes the plan and the size
    assert _lib.workspace_bytes(_shape(T=65536, H=16, seg=1)) > f


@pytest.mark.parametrize("T,B,H,D", [(1, 1, 4, 128), (64, 2, 3, 64), (37, 1, 16, 128)])
def test_one_block_bf16_chunk_sizes(T, B, H, D):
    """A bf16 chunk of one 64-token block runs on the fp32 kernels: its saved
    buffer is the fp32 chunk's, and its workspaces are the fp32 chunk's plus
    fp32 copies of its token tensors (q, k, v, o forward; q, k, v, dO, dq,
    dk, dv backward), each rounded up to 256 bytes.  Two blocks stay bf16."""
    bf, f32 = _lib.Shape(B, T, H, D, D, 1, 0), _lib.Shape(B, T, H, D, D, 0, 0)
    copy = -(-(B * T * H * D * 4) // 256) * 256
    assert _lib.saved_bytes(bf) == _lib.saved_bytes(f32)
    assert _lib.workspace_bytes(bf) == _lib.workspace_bytes(f32) + 4 * copy
    assert _lib.workspace_bytes(bf, backward=True) == \
        _lib.workspace_bytes(f32, backward=True) + 7 * copy
    two = _lib.Shape(B, 65, H, D, D, 1, 0)
    assert _lib.saved_bytes(two) < _lib.saved_bytes(_lib.Shape(B, 65, H, D, D, 0, 0))


@pytest.mark.parametrize("T,N,alpha", [(262144, 8, 0.5), (262144, 8, 0.0), (262144, 8, 1.0),
                                       (131072, 4, 0.75), (65536, 16, 0.25)])
def test_planner_matches_oracle_search(T, N, alpha):
    from oracle import plan as op
    assert chunk_lengths(T, N, alpha) == op.skewed_lengths(T, N, alpha, 1.0, 0.25, 64)


def _cshape(B=1, T=128, C=64, W=4, dtype=1, act=0):
    return _lib.ConvShape(B, T, C, W, dtype, act)


def _conv_fwd(shape, x=1 * G, w=2 * G, cin=None, y=3 * G, cout=4 * G):
    L = _lib.load()
    vp = lambda p: None if p is None else ctypes.c_void_p(p)
    return L.sf_gdn_shortconv_fwd(ctypes.byref(shape), vp(x), vp(w), vp(cin), vp(y), vp(cout),
                                  None)


@pytest.mark.parametrize("shape,code", [
    (_cshape(W=0), _lib.SF_ERR_UNSUPPORTED),
    (_cshape(W=9), _lib.SF_ERR_UNSUPPORTED),
    (_cshape(C=12), _lib.SF_ERR_UNSUPPORTED),
    (_cshape(act=2), _lib.SF_ERR_INVALID_ARG),
    (_cshape(B=0), _lib.SF_ERR_INVALID_ARG),
    (_cshape(T=-1), _lib.SF_ERR_INVALID_ARG),
    (_cshape(dtype=5), _lib.SF_ERR_INVALID_ARG),
])
def test_conv_rejects_bad_shapes(shape, code):
    assert _conv_fwd(shape) == code


def test_conv_rejects_missing_overlapping_and_small_workspace():
    assert _conv_fwd(_cshape(), x=None) == _lib.SF_ERR_INVALID_ARG
    assert _conv_fwd(_cshape(), w=None) == _lib.SF_ERR_INVALID_ARG
    assert _conv_fwd(_cshape(), y=G + 64) == _lib.SF_ERR_INVALID_ARG        # y overlaps x
    assert _conv_fwd(_cshape(), cout=3 * G + 64) == _lib.SF_ERR_INVALID_ARG  # overlaps y
    assert _conv_fwd(_cshape(), x=G + 8) == _lib.SF_ERR_INVALID_ARG         # misaligned
    shape = _cshape(T=4096, C=256)
    need = _lib.shortconv_bwd_workspace_bytes(shape)
    assert need > 0
    L = _lib.load()
    vp = lambda p: None if p is None else ctypes.c_void_p(p)
    args = [vp(1 * G), vp(2 * G), None, vp(3 * G), None, vp(4 * G), vp(5 * G), vp(6 * G)]
    assert L.sf_gdn_shortconv_bwd(ctypes.byref(shape), *args, vp(8 * G), ctypes.c_size_t(need - 1),
                                  None) == _lib.SF_ERR_WORKSPACE
    assert L.sf_gdn_shortconv_bwd(ctypes.byref(shape), *args, None, ctypes.c_size_t(0),
                                  None) == _lib.SF_ERR_WORKSPACE


def test_split_calls_reject_unknown_phase():
    L = _lib.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    shape = _shape(T=8192, H=2)
    st = L.sf_gdn_chunk_fwd_split(ctypes.byref(shape), vp(1 * G), vp(2 * G), vp(3 * G), vp(4 * G),
                                  vp(5 * G), None, vp(6 * G), vp(7 * G), None, ctypes.c_size_t(0),
                                  vp(24 * G), ctypes.c_size_t(_lib.workspace_bytes(shape)), 7, None)
    assert st == _lib.SF_ERR_INVALID_ARG
    assert "phase" in L.sf_last_error_message().decode()
    st = L.sf_gdn_chunk_bwd_saved_split(ctypes.byref(shape), vp(1 * G), vp(2 * G), vp(3 * G),
                                        vp(4 * G), vp(5 * G), vp(20 * G),
                                        ctypes.c_size_t(_lib.saved_bytes(shape)), vp(6 * G), None,
                                        vp(8 * G), vp(9 * G), vp(10 * G), vp(11 * G), vp(12 * G),
                                        None, vp(24 * G),
                                        ctypes.c_size_t(_lib.workspace_bytes(shape, backward=True)),
                                        -1, None)
    assert st == _lib.SF_ERR_INVALID_ARG


def test_bench_algorithmic_figures():
    """The benchmark's per-kernel models against the method's per-token-head
    figures at d = 128, block C = 64: bytes fwd 4 d * 2 + 8 = 1,032 and bwd
    7 d * 2 + 16 = 1,808 (bf16 activations, fp32 gates); the forward output
    kernel's matrix products 2 C (3 d + 2 d) + 6 d^2 = 180,224 flop (the
    forward's 182,955 without the triangular solve's (2/3) C^2, which is not
    an MFMA product)."""
    import bench
    assert bench.kernel_bytes_per_token_head("gdn_bwd_grads", 128) == 1808
    assert bench.kernel_bytes_per_token_head("gdn_fwd_out", 128) == 1032
    assert bench.kernel_bytes_per_token_head("gdn_fwd_summary", 128) is None
    assert bench.kernel_flops_per_block("gdn_fwd_out", 128) / 64 == 180224


def test_kernel_labels():
    """Profiler kernel names (mangled and demangled) map to the launch labels
    the profiles and traffic figures use, for every form of a kernel."""
    import bench
    lab = bench.kernel_label
    assert lab("_ZN5sfgdn21gdn_bwd_dscan2_kernelIDF16bLi128ELb1EEEvNS_7BwdArgsEiiPKfi") == "gdn_bwd_dscan"
    assert lab("_ZN5sfgdn21gdn_bwd_dscan2_kernelIDF16bLi128ELb0EEEvNS_7BwdArgsEiiPKfi") == "gdn_bwd_dscan_summary"
    assert lab("_ZN5sfgdn20gdn_bwd_dscan_kernelIfLi64ELb1EEEvNS_7BwdArgsEiiPKfi") == "gdn_bwd_dscan"
    assert lab("void sfgdn::gdn_bwd_dscan2_kernel<__bf16, 128, false>(sfgdn::BwdArgs, int, int, float const*, int)") == "gdn_bwd_dscan_summary"
    assert lab("_ZN5sfgdn23gdn_fwd_summary2_kernelIDF16bLi128EEEvNS_7FwdArgsEi") == "gdn_fwd_summary"
    assert lab("_ZN5sfgdn22gdn_fwd_summary_kernelIfLi64EEEvNS_7FwdArgsEi") == "gdn_fwd_summary"
    assert lab("_ZN5sfgdn19gdn_fwd_out2_kernelIDF16bLi128ELi2EEEvNS_7FwdArgsEPT_") == "gdn_fwd_out_save"
    assert lab("_ZN5sfgdn20gdn_bwd_grads_kernelIDF16bLi128EEEvNS_7BwdArgsE") == "gdn_bwd_grads"
    assert lab("_ZN5sfgdn16gdn_chain_kernelILi128ELb1EEEvNS_9ChainArgsE") == "gdn_chain_bwd"
    assert lab("elementwise_kernel") is None


def test_segment_plan():
    """The in-chunk scan's segments: enough to occupy 256 compute units, no
    shorter than about sqrt(0.3 nblk) blocks, an explicit length honoured,
    none for an empty chunk."""
    plan = lambda T, H, seg=0: _lib.segment_plan(_shape(T=T, H=H, seg=seg))
    assert plan(65536, 16) == (64, 16)      # 16 heads x 16 segments
    assert plan(62720, 16) == (62, 16)      # ragged last segment
    assert plan(16384, 16) == (16, 16)
    assert plan(65536, 32) == (128, 8)
    assert plan(1024, 16) == (2, 8)         # short chunk: floor sqrt(0.3 * 16) ~ 2
    assert plan(256, 2) == (1, 4)
    assert plan(64, 16) == (1, 1)
    assert plan(1024, 16, seg=1) == (1, 16)
    assert plan(1024, 16, seg=64) == (16, 1)  # clamped to the chunk
    assert plan(0, 16) == (1, 0)


def test_rejects_plans_beyond_the_chain_kernels_range():
    """The chain kernels address one sequence's segment maps through a
    32-bit byte range: P * D * D * 4 bytes must fit, so an explicit one-block
    segment on a chunk of 2,097,152 tokens at D = 128 (32,768 segments) is
    refused on the host, and the default plan for the same chunk is not."""
    big = 32768 * 64
    L, P = ctypes.c_int(0), ctypes.c_int(0)
    lib = _lib.load()
    s = _shape(T=big, H=1, seg=1)
    assert lib.sf_gdn_segment_plan(ctypes.byref(s), ctypes.byref(L), ctypes.byref(P)) == \
        _lib.SF_ERR_UNSUPPORTED
    assert "segments" in lib.sf_last_error_message().decode()
    assert _lib.segment_plan(_shape(T=big - 64, H=1, seg=1)) == (1, 32767)
    assert _lib.segment_plan(_shape(T=big, H=1))[1] < 32768


_NO_GPU_CALL = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from linear_recurrence_chunked_gated_amd import _lib
G = 1 << 30
L = _lib.load()
vp = lambda x: None if x is None else ctypes.c_void_p(x)
shape = _lib.Shape(1, 128, 2, 128, 128, 1, 0)
ws = _lib.workspace_bytes(shape)
st = L.sf_gdn_chunk_fwd(ctypes.byref(shape), vp(G), vp(2 * G), vp(3 * G), vp(4 * G), vp(5 * G),
                        None, vp(6 * G), vp(7 * G), vp(16 * G), ctypes.c_size_t(ws), None)
print(st, L.sf_last_error_message().decode())
"""


def test_hip_failure_is_a_status():
    """A call whose arguments pass the host checks but whose HIP calls fail
    returns SF_ERR_HIP with the HIP error text; nothing aborts.  Run in a
    child process that can see no GPU (ROCR_VISIBLE_DEVICES and
    HIP_VISIBLE_DEVICES empty), so the failure is the runtime's own and no
    kernel can ever run on the placeholder pointers."""
    import subprocess
    import sys
    env = dict(os.environ, ROCR_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="",
               CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", _NO_GPU_CALL, ROOT], capture_output=True, text=True,
                       env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    line = r.stdout.strip().splitlines()[-1]
    code, msg = line.split(" ", 1)
    assert int(code) == _lib.SF_ERR_HIP, line
    assert msg, line


def test_split_lengths():
    """The split at fraction f: each chunk into two parts of whole 64-token
    blocks, the first about f of it; order and total preserved; chunks of
    one block stay whole; f outside (0, 1) is refused."""
    from linear_recurrence_chunked_gated_amd.chain import split_lengths
    L = chunk_lengths(262144, 8, 0.5)
    for f in (0.3, 0.5, 0.7, 0.9):
        parts = split_lengths(L, f)
        assert len(parts) == 2 * len(L) and sum(parts) == sum(L)
        assert all(p > 0 and p % 64 == 0 for p in parts)
        for i, n in enumerate(L):
            assert parts[2 * i] + parts[2 * i + 1] == n
            assert abs(parts[2 * i] - f * n) <= 32
    assert split_lengths([64, 128], 0.5) == [64, 64, 64]
    with pytest.raises(ValueError):
        split_lengths(L, 1.0)
