// C ABI of the chunked gated delta-rule library: argument checks, the
// segment plan, workspace carving and kernel launches on the caller's stream.
#include <cmath>
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <string>
#include <vector>

#include "../../include/sf_gdn.h"
#include "gdn_kernels.hpp"

namespace sfgdn {
hipError_t launch_copy_state(float* dst, const float* src, size_t n, hipStream_t st);
// n elements between bf16 and fp32 (n a multiple of 8)
hipError_t launch_cast_to_f32(float* dst, const void* src, size_t n, hipStream_t st);
hipError_t launch_cast_to_bf16(void* dst, const float* src, size_t n, hipStream_t st);
}

using namespace sfgdn;

namespace {

thread_local std::string g_err;

sf_status fail(sf_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int B, T, H, D, dtype;
  int nblk, L, P;
  size_t state_elem;  // bytes per stored per-block state element (bwd)
  // A bf16 chunk of one block (T <= 64) runs on the fp32 kernels, on fp32
  // copies of its token tensors in the workspace, and its outputs are rounded
  // to bf16 at the end.  Such a chunk costs next to nothing either way, and
  // in fp32 its gradients keep their accuracy where a one- or two-token
  // chunk's gate gradients, single sums with heavy cancellation, lose it to
  // the rounding of bf16 operands.
  bool up;
};

sf_status make_plan(const sf_gdn_shape* s, Plan& p) {
  if (!s) return fail(SF_ERR_INVALID_ARG, "shape is NULL");
  if (s->B <= 0 || s->H <= 0 || s->T < 0 || s->Dk <= 0 || s->Dv <= 0)
    return fail(SF_ERR_INVALID_ARG, "dimensions must be positive (T may be 0)");
  if (s->dtype != SF_DTYPE_F32 && s->dtype != SF_DTYPE_BF16)
    return fail(SF_ERR_INVALID_ARG, "unknown dtype");
  if (s->seg_blocks < 0) return fail(SF_ERR_INVALID_ARG, "seg_blocks must be >= 0");
  if (s->Dk != s->Dv) return fail(SF_ERR_UNSUPPORTED, "Dk != Dv is not supported");
  if (s->Dk != 64 && s->Dk != 128) return fail(SF_ERR_UNSUPPORTED, "Dk must be 64 or 128");
  if ((long long)s->B * s->H > (1LL << 20))
    return fail(SF_ERR_UNSUPPORTED, "B*H too large");
  p.B = s->B;
  p.T = s->T;
  p.H = s->H;
  p.D = s->Dk;
  p.dtype = s->dtype;
  p.nblk = (s->T + BLK - 1) / BLK;
  if (p.nblk == 0) {
    p.L = 1;
    p.P = 0;
  } else {
    int L = s->seg_blocks;
    if (L == 0) {
      // Enough segments that B*H*P workgroups cover the 256 compute units,
      // but no shorter than about sqrt(0.3 nblk) blocks: each segment adds
      // one dependent step to the chain (about 2 us), each block of
      // segment length about 7 us to the summary and output passes, so on
      // short chunks, where 256 workgroups cannot be filled with whole
      // work anyway, the sum of the two is smallest there.
      const long long bh = (long long)s->B * s->H;
      long long P0 = (256 + bh - 1) / bh;
      if (P0 > p.nblk) P0 = p.nblk;
      if (P0 < 1) P0 = 1;
      L = (int)((p.nblk + P0 - 1) / P0);
      const int Lmin = (int)std::lround(std::sqrt(0.3 * (double)p.nblk));
      if (L < Lmin) L = Lmin;
    }
    if (L > p.nblk) L = p.nblk;
    p.L = L;
    p.P = (p.nblk + L - 1) / L;
    if ((long long)p.B * p.H * p.P > (1LL << 30))
      return fail(SF_ERR_UNSUPPORTED, "too many segments");
    // The chain kernels address one sequence's P segment maps through a
    // buffer resource with a 32-bit byte range.
    if ((unsigned long long)p.P * p.D * p.D * sizeof(float) > 0x7fffffffULL)
      return fail(SF_ERR_UNSUPPORTED,
                  "too many segments per sequence for the chain kernels (raise seg_blocks)");
  }
  // per-block states and state gradients are stored in the operand type (the
  // precision in which they enter every product that reads them)
  p.state_elem = p.dtype == SF_DTYPE_BF16 ? 2 : 4;
  p.up = p.dtype == SF_DTYPE_BF16 && p.nblk == 1;
  return SF_OK;
}

size_t dd(const Plan& p) { return (size_t)p.D * p.D; }
size_t seg_buf(const Plan& p) { return align_up((size_t)p.B * p.H * p.P * dd(p) * sizeof(float)); }
size_t elem(const Plan& p) { return p.dtype == SF_DTYPE_BF16 ? 2 : 4; }
// per-block Tpp = T diag(beta) of the Pre kernel: [B*H][nblk][64][64] in the operand type
size_t tw_buf(const Plan& p) {
  return align_up((size_t)p.B * p.H * p.nblk * BLK * BLK * elem(p));  // Tpp per block
}
size_t fwd_seg(const Plan& p) { return p.P > 1 ? 3 * seg_buf(p) : 0; }
// The plan the kernels run (fp32 for an upcast chunk) and the size of one
// fp32 copy of a token tensor.
Plan kplan(const Plan& p) {
  Plan k = p;
  if (p.up) {
    k.dtype = SF_DTYPE_F32;
    k.state_elem = 4;
    k.up = false;
  }
  return k;
}
size_t tok_f32(const Plan& p) { return align_up((size_t)p.B * p.T * p.H * p.D * 4); }
// kernel workspaces of a plan (the kernels' dtype)
size_t fwd_core(const Plan& p) { return fwd_seg(p) + tw_buf(p); }
size_t blk_buf(const Plan& p) { return align_up((size_t)p.B * p.H * p.nblk * dd(p) * p.state_elem); }
// per-block Vn of the state-storing forward: [B*H][nblk][64 x D] in the operand type
size_t vn_buf(const Plan& p) { return align_up((size_t)p.B * p.H * p.nblk * BLK * p.D * elem(p)); }
// the gradient kernel's global tile areas (fp32 at d = 128)
size_t far_buf(const Plan& p) { return align_up(bwd_far_bytes(p.dtype == SF_DTYPE_F32, p.D)); }
size_t bwd_core(const Plan& p) {
  if (p.P == 0) return 0;
  return 3 * seg_buf(p) + 3 * seg_buf(p) + 2 * blk_buf(p) + tw_buf(p) + vn_buf(p) + far_buf(p);
}
// caller workspaces: an upcast chunk adds fp32 copies of q, k, v, o (forward)
// or q, k, v, dO, dq, dk, dv (backward) after the kernels' workspace
size_t fwd_ws(const Plan& p) { return p.up ? fwd_core(kplan(p)) + 4 * tok_f32(p) : fwd_core(p); }
size_t bwd_ws(const Plan& p) { return p.up ? bwd_core(kplan(p)) + 7 * tok_f32(p) : bwd_core(p); }

struct Range {
  const void* p;
  size_t n;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

sf_status check_ptrs(const std::vector<Range>& in, const std::vector<Range>& out,
                     const std::vector<const char*>& required) {
  (void)required;
  for (const Range& r : in)
    if (r.p && ((uintptr_t)r.p % 16)) return fail(SF_ERR_INVALID_ARG, std::string(r.name) + " is not 16-byte aligned");
  for (const Range& r : out)
    if (r.p && ((uintptr_t)r.p % 16)) return fail(SF_ERR_INVALID_ARG, std::string(r.name) + " is not 16-byte aligned");
  for (size_t i = 0; i < out.size(); ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r))
        return fail(SF_ERR_INVALID_ARG, std::string(out[i].name) + " overlaps input " + r.name);
    for (size_t j = i + 1; j < out.size(); ++j)
      if (overlap(out[i], out[j]))
        return fail(SF_ERR_INVALID_ARG, std::string(out[i].name) + " overlaps output " + out[j].name);
  }
  return SF_OK;
}

// ------------------------------------------------------------ profiler ----
struct ProfRec {
  const char* name;
  int ev;
};

}  // namespace

namespace sfgdn {
struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> ev;
  std::vector<ProfRec> recs;
  int open = -1;
  std::vector<std::string> names;
  std::vector<long long> counts;
  std::vector<double> ms;
};

void prof_begin(Profiler* p, const char* name, hipStream_t st) {
  if (!p) return;
  p->open = -1;
  const int idx = (int)p->recs.size() * 2;
  if (idx + 2 > (int)p->ev.size()) return;
  if (hipEventRecord(p->ev[idx], st) != hipSuccess) return;
  p->recs.push_back(ProfRec{name, idx});
  p->open = idx;
}

void prof_end(Profiler* p, hipStream_t st) {
  if (!p || p->open < 0) return;
  if (hipEventRecord(p->ev[p->open + 1], st) != hipSuccess) p->recs.pop_back();
  p->open = -1;
}
}  // namespace sfgdn

namespace {
Profiler g_prof;

Profiler* prof_if_on() { return g_prof.on.load(std::memory_order_acquire) ? &g_prof : nullptr; }

// A call records its launches only while profiling is on, under the
// profiler's lock (begin/end take it too); otherwise it runs unlocked.
template <typename F>
sf_status run_locked(F f) {
  if (g_prof.on.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    return f(prof_if_on());
  }
  return f(nullptr);
}

sf_status hip_fail(hipError_t e, const char* what) {
  return fail(SF_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

// ---------------------------------------------------------------- ABI ------
extern "C" {

sf_status sf_gdn_segment_plan(const sf_gdn_shape* shape, int* seg_blocks, int* segments) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  if (!seg_blocks || !segments) return fail(SF_ERR_INVALID_ARG, "output pointer is NULL");
  *seg_blocks = p.L;
  *segments = p.P;
  return SF_OK;
}

sf_status sf_gdn_chunk_fwd_workspace_size(const sf_gdn_shape* shape, size_t* bytes) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  if (!bytes) return fail(SF_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = fwd_ws(p);
  return SF_OK;
}

sf_status sf_gdn_chunk_bwd_workspace_size(const sf_gdn_shape* shape, size_t* bytes) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  if (!bytes) return fail(SF_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_ws(p);
  return SF_OK;
}

}  // extern "C"

namespace {

// Layout: per-block entry states [B*H*nblk][D][D], the segment maps
// [B*H*P][D][D] row-major (P > 1), then the Pre kernel's per-block Tpp.
size_t saved_maps_off(const Plan& p) { return blk_buf(p); }
size_t saved_tw_off(const Plan& p) { return blk_buf(p) + (p.P > 1 ? seg_buf(p) : 0); }
size_t saved_vn_off(const Plan& p) { return saved_tw_off(p) + tw_buf(p); }
// laid out for the kernels' plan (an upcast chunk saves fp32)
size_t saved_bytes(const Plan& p) {
  if (p.P == 0) return 0;
  const Plan k = kplan(p);
  return saved_vn_off(k) + vn_buf(k);
}

// Forward; with `saved` it also stores the per-block entry states, all
// segment maps, the per-block Tpp and the per-block Vn there.
sf_status fwd_impl(const sf_gdn_shape* shape, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* S_in, void* o,
                   float* S_out, void* saved, size_t sv_bytes, void* workspace, size_t ws_bytes,
                   void* stream, bool save, int phase = PHASE_ALL) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  const size_t ntok = (size_t)p.B * p.T * p.H;
  const size_t nst = (size_t)p.B * p.H * dd(p);
  if (p.T > 0 && (!q || !k || !v || !alpha || !beta || !o))
    return fail(SF_ERR_INVALID_ARG, "q, k, v, alpha, beta and o are required");
  std::vector<Range> in = {{q, ntok * p.D * elem(p), "q"},     {k, ntok * p.D * elem(p), "k"},
                           {v, ntok * p.D * elem(p), "v"},     {alpha, ntok * 4, "alpha"},
                           {beta, ntok * 4, "beta"},           {S_in, nst * 4, "S_in"},
                           {workspace, ws_bytes, "workspace"}};
  std::vector<Range> out = {{o, ntok * p.D * elem(p), "o"}, {S_out, nst * 4, "S_out"}};
  if (save) out.push_back({saved, sv_bytes, "saved"});
  if ((s = check_ptrs(in, out, {})) != SF_OK) return s;
  if (save) {
    const size_t sneed = saved_bytes(p);
    if (sneed > 0 && (!saved || sv_bytes < sneed))
      return fail(SF_ERR_INVALID_ARG, "saved buffer needs " + std::to_string(sneed) + " bytes");
    if (saved && ((uintptr_t)saved % kAlign))
      return fail(SF_ERR_INVALID_ARG, "saved buffer is not 256-byte aligned");
  }
  const size_t need = fwd_ws(p);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(SF_ERR_WORKSPACE, "forward workspace needs " + std::to_string(need) + " bytes");
  if (workspace && ((uintptr_t)workspace % kAlign))
    return fail(SF_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;

  return run_locked([&](Profiler* prof) -> sf_status {
    if (p.T == 0) {
      if (S_out && phase != PHASE_BEGIN) {
        hipError_t e = launch_copy_state(S_out, S_in, nst, st);
        if (e != hipSuccess) return hip_fail(e, "state copy");
      }
      return SF_OK;
    }
    const Plan kp = kplan(p);
    char* ws = (char*)workspace;
    const void *kq = q, *kk = k, *kv = v;
    void* ko = o;
    float* up = nullptr;  // fp32 copies of q, k, v, o (upcast chunk)
    hipError_t e;
    if (p.up) {
      char* base = ws + fwd_core(kp);
      float* c[4];
      for (int i = 0; i < 4; ++i) c[i] = (float*)(base + i * tok_f32(p));
      if (phase != PHASE_END) {
        const void* src[3] = {q, k, v};
        for (int i = 0; i < 3; ++i)
          if ((e = launch_cast_to_f32(c[i], src[i], ntok * p.D, st)) != hipSuccess)
            return hip_fail(e, "input cast");
      }
      kq = c[0]; kk = c[1]; kv = c[2]; ko = c[3];
      up = c[3];
    }
    FwdArgs a{};
    a.q = kq; a.k = kk; a.v = kv; a.alpha = alpha; a.beta = beta; a.S_in = S_in;
    a.o = ko; a.S_out = S_out;
    a.B = p.B; a.T = p.T; a.H = p.H; a.nblk = p.nblk; a.L = p.L; a.P = p.P;
    void* hsave = save ? saved : nullptr;
    a.tw = save ? (char*)saved + saved_tw_off(kp) : ws + fwd_seg(kp);
    a.vst = save ? (char*)saved + saved_vn_off(kp) : nullptr;
    if (p.P > 1) {
      a.Mseg = (float*)ws;
      a.MBseg = save ? (float*)((char*)saved + saved_maps_off(kp)) : nullptr;
      a.Nseg = (float*)(ws + seg_buf(kp));
      a.Sst = (float*)(ws + 2 * seg_buf(kp));
      a.sst_P = p.P;
    } else {
      a.Sst = S_in;
      a.sst_P = 1;
    }
    if (kp.dtype == SF_DTYPE_BF16)
      e = (p.D == 128) ? launch_fwd<bf16, 128>(a, hsave, phase, st, prof)
                       : launch_fwd<bf16, 64>(a, hsave, phase, st, prof);
    else
      e = (p.D == 128) ? launch_fwd<float, 128>(a, hsave, phase, st, prof)
                       : launch_fwd<float, 64>(a, hsave, phase, st, prof);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    if (up && phase != PHASE_BEGIN &&
        (e = launch_cast_to_bf16(o, up, ntok * p.D, st)) != hipSuccess)
      return hip_fail(e, "output cast");
    return SF_OK;
  });
}

// Backward; with `saved` (from fwd_impl with save) the forward recompute is
// skipped and S_in is not needed.
sf_status bwd_impl(const sf_gdn_shape* shape, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* S_in, const void* saved,
                   size_t sv_bytes, const void* dO, const float* dS_out, void* dq, void* dk,
                   void* dv, float* dalpha, float* dbeta, float* dS_in, void* workspace,
                   size_t ws_bytes, void* stream, bool use_saved, int phase = PHASE_ALL) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  const size_t ntok = (size_t)p.B * p.T * p.H;
  const size_t nst = (size_t)p.B * p.H * dd(p);
  const size_t nt = ntok * p.D * elem(p);
  if (p.T > 0 && (!q || !k || !v || !alpha || !beta || !dO || !dq || !dk || !dv || !dalpha || !dbeta))
    return fail(SF_ERR_INVALID_ARG, "q, k, v, alpha, beta, dO, dq, dk, dv, dalpha and dbeta are required");
  std::vector<Range> in = {{q, nt, "q"},          {k, nt, "k"},           {v, nt, "v"},
                           {alpha, ntok * 4, "alpha"}, {beta, ntok * 4, "beta"}, {S_in, nst * 4, "S_in"},
                           {dO, nt, "dO"},        {dS_out, nst * 4, "dS_out"},
                           {workspace, ws_bytes, "workspace"}};
  if (use_saved) in.push_back({saved, sv_bytes, "saved"});
  std::vector<Range> out = {{dq, nt, "dq"}, {dk, nt, "dk"}, {dv, nt, "dv"}, {dalpha, ntok * 4, "dalpha"},
                            {dbeta, ntok * 4, "dbeta"}, {dS_in, nst * 4, "dS_in"}};
  if ((s = check_ptrs(in, out, {})) != SF_OK) return s;
  if (use_saved) {
    const size_t sneed = saved_bytes(p);
    if (sneed > 0 && (!saved || sv_bytes < sneed))
      return fail(SF_ERR_INVALID_ARG, "saved buffer needs " + std::to_string(sneed) + " bytes");
    if (saved && ((uintptr_t)saved % kAlign))
      return fail(SF_ERR_INVALID_ARG, "saved buffer is not 256-byte aligned");
  }
  const size_t need = bwd_ws(p);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(SF_ERR_WORKSPACE, "backward workspace needs " + std::to_string(need) + " bytes");
  if (workspace && ((uintptr_t)workspace % kAlign))
    return fail(SF_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;

  return run_locked([&](Profiler* prof) -> sf_status {
    if (p.T == 0) {
      if (dS_in && phase != PHASE_BEGIN) {
        hipError_t e = launch_copy_state(dS_in, dS_out, nst, st);
        if (e != hipSuccess) return hip_fail(e, "state copy");
      }
      return SF_OK;
    }
    const Plan kp = kplan(p);
    char* ws = (char*)workspace;
    const void *kq = q, *kk = k, *kv = v, *kdo = dO;
    void *kdq = dq, *kdk = dk, *kdv = dv;
    float* up = nullptr;  // fp32 copies of q, k, v, dO, dq, dk, dv (upcast chunk)
    hipError_t e;
    if (p.up) {
      char* base = ws + bwd_core(kp);
      float* c[7];
      for (int i = 0; i < 7; ++i) c[i] = (float*)(base + i * tok_f32(p));
      if (phase != PHASE_END) {
        const void* src[4] = {q, k, v, dO};
        for (int i = 0; i < 4; ++i)
          if ((e = launch_cast_to_f32(c[i], src[i], ntok * p.D, st)) != hipSuccess)
            return hip_fail(e, "input cast");
      }
      kq = c[0]; kk = c[1]; kv = c[2]; kdo = c[3];
      kdq = c[4]; kdk = c[5]; kdv = c[6];
      up = c[4];
    }
    BwdArgs a{};
    FwdArgs& f = a.f;
    f.q = kq; f.k = kk; f.v = kv; f.alpha = alpha; f.beta = beta; f.S_in = S_in;
    f.o = nullptr; f.S_out = nullptr;
    f.B = p.B; f.T = p.T; f.H = p.H; f.nblk = p.nblk; f.L = p.L; f.P = p.P;
    const size_t sb = seg_buf(kp), bb = blk_buf(kp);
    f.Mseg = (float*)ws;
    f.Nseg = (float*)(ws + sb);
    f.Sst = (float*)(ws + 2 * sb);
    f.sst_P = p.P;
    a.NBseg = (float*)(ws + 3 * sb);
    a.dSend = (float*)(ws + 4 * sb);
    a.hst = ws + 5 * sb;
    a.dhst = ws + 5 * sb + bb;
    f.tw = ws + 5 * sb + 2 * bb;
    f.MBseg = (float*)(ws + 5 * sb + 2 * bb + tw_buf(kp));
    f.vst = ws + 6 * sb + 2 * bb + tw_buf(kp);
    a.far = far_buf(kp) ? ws + 6 * sb + 2 * bb + tw_buf(kp) + vn_buf(kp) : nullptr;
    if (use_saved) {
      char* sv = (char*)const_cast<void*>(saved);
      a.hst = sv;
      if (p.P > 1) f.MBseg = (float*)(sv + saved_maps_off(kp));
      f.tw = sv + saved_tw_off(kp);
      f.vst = sv + saved_vn_off(kp);
    }
    a.dO = kdo; a.dS_out = dS_out;
    a.dq = kdq; a.dk = kdk; a.dv = kdv; a.dalpha = dalpha; a.dbeta = dbeta; a.dS_in = dS_in;
    if (kp.dtype == SF_DTYPE_BF16)
      e = (p.D == 128) ? launch_bwd<bf16, 128>(a, use_saved, phase, st, prof)
                       : launch_bwd<bf16, 64>(a, use_saved, phase, st, prof);
    else
      e = (p.D == 128) ? launch_bwd<float, 128>(a, use_saved, phase, st, prof)
                       : launch_bwd<float, 64>(a, use_saved, phase, st, prof);
    if (e == hipErrorNotSupported) return fail(SF_ERR_UNSUPPORTED, "backward not available");
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    if (up && phase != PHASE_BEGIN) {
      void* dst[3] = {dq, dk, dv};
      for (int i = 0; i < 3; ++i)
        if ((e = launch_cast_to_bf16(dst[i], up + i * (tok_f32(p) / 4), ntok * p.D, st)) !=
            hipSuccess)
          return hip_fail(e, "output cast");
    }
    return SF_OK;
  });
}

}  // namespace

namespace {

// ------------------------------------------------------- short convolution
struct ConvPlan {
  int B, T, C, W, dtype, act;
  int GR, nrun;  // backward: tokens per run, runs per sequence
};

sf_status make_conv_plan(const sf_conv_shape* s, ConvPlan& p) {
  if (!s) return fail(SF_ERR_INVALID_ARG, "shape is NULL");
  if (s->B <= 0 || s->T < 0 || s->C <= 0)
    return fail(SF_ERR_INVALID_ARG, "B and C must be positive and T >= 0");
  if (s->dtype != SF_DTYPE_F32 && s->dtype != SF_DTYPE_BF16)
    return fail(SF_ERR_INVALID_ARG, "unknown dtype");
  if (s->W < 1 || s->W > 8) return fail(SF_ERR_UNSUPPORTED, "W must be in 1..8");
  if (s->act != 0 && s->act != 1) return fail(SF_ERR_INVALID_ARG, "act must be 0 or 1");
  if (s->C % 8) return fail(SF_ERR_UNSUPPORTED, "C must be a multiple of 8");
  if ((long long)s->B * s->T * s->C > (1LL << 40)) return fail(SF_ERR_UNSUPPORTED, "too large");
  p.B = s->B; p.T = s->T; p.C = s->C; p.W = s->W; p.dtype = s->dtype; p.act = s->act;
  // Backward runs: about 1024 (channel group, run, b) workgroups, four per
  // compute unit, at least 32 tokens each.  Fewer, longer runs cut the
  // weight-gradient partials (one per run, reduced afterwards) and the per-run
  // halo; twice as many runs cost more in that reduction, half as many left
  // compute units idle.
  const long long gx = (s->C / (s->dtype == SF_DTYPE_BF16 ? 4 : 2) + 255) / 256;
  long long want = (1024 + gx * s->B - 1) / (gx * s->B);
  if (want < 1) want = 1;
  long long GR = s->T > 0 ? (s->T + want - 1) / want : 16;
  GR = (GR + 15) / 16 * 16;
  if (GR < 32) GR = 32;
  p.GR = (int)GR;
  p.nrun = s->T > 0 ? (int)((s->T + GR - 1) / GR) : 0;
  return SF_OK;
}

size_t conv_bwd_ws(const ConvPlan& p) {
  const size_t np = (size_t)p.B * p.nrun, ng = (np + 31) / 32;  // partials, group sums
  return align_up((np + ng) * p.C * p.W * sizeof(float));
}

}  // namespace

extern "C" {

sf_status sf_gdn_chunk_fwd(const sf_gdn_shape* shape, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S_in, void* o,
                           float* S_out, void* workspace, size_t ws_bytes, void* stream) {
  return fwd_impl(shape, q, k, v, alpha, beta, S_in, o, S_out, nullptr, 0, workspace, ws_bytes,
                  stream, false);
}

sf_status sf_gdn_chunk_bwd(const sf_gdn_shape* shape, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S_in,
                           const void* dO, const float* dS_out, void* dq, void* dk, void* dv,
                           float* dalpha, float* dbeta, float* dS_in, void* workspace,
                           size_t ws_bytes, void* stream) {
  return bwd_impl(shape, q, k, v, alpha, beta, S_in, nullptr, 0, dO, dS_out, dq, dk, dv, dalpha,
                  dbeta, dS_in, workspace, ws_bytes, stream, false);
}

sf_status sf_gdn_chunk_saved_size(const sf_gdn_shape* shape, size_t* bytes) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  if (!bytes) return fail(SF_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = saved_bytes(p);
  return SF_OK;
}

sf_status sf_gdn_chunk_fwd_save(const sf_gdn_shape* shape, const void* q, const void* k,
                                const void* v, const float* alpha, const float* beta,
                                const float* S_in, void* o, float* S_out, void* saved,
                                size_t saved_bytes_, void* workspace, size_t ws_bytes,
                                void* stream) {
  return fwd_impl(shape, q, k, v, alpha, beta, S_in, o, S_out, saved, saved_bytes_, workspace,
                  ws_bytes, stream, true);
}

sf_status sf_gdn_chunk_bwd_saved(const sf_gdn_shape* shape, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const void* saved, size_t saved_bytes_, const void* dO,
                                 const float* dS_out, void* dq, void* dk, void* dv, float* dalpha,
                                 float* dbeta, float* dS_in, void* workspace, size_t ws_bytes,
                                 void* stream) {
  return bwd_impl(shape, q, k, v, alpha, beta, nullptr, saved, saved_bytes_, dO, dS_out, dq, dk,
                  dv, dalpha, dbeta, dS_in, workspace, ws_bytes, stream, true);
}

// ------------------------------------------------ no-allocation forward ----
// Workspace of sf_gdn_chunk_fwd_noalloc: one static device array per GPU,
// held until the process ends.  Host code never uses the array's name as an
// address: each device's copy is looked up once (hipGetSymbolAddress, with
// that device current) and that pointer is what the kernels get.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // by device ordinal; null until looked up

sf_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SF_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SF_OK;
}
}  // namespace

sf_status sf_gdn_chunk_fwd_noalloc(const sf_gdn_shape* shape, const void* q, const void* k,
                                   const void* v, const float* alpha, const float* beta,
                                   const float* S_in, void* o, float* S_out, void* stream) {
  Plan p;
  sf_status s = make_plan(shape, p);
  if (s != SF_OK) return s;
  const size_t need = fwd_ws(p);
  if (need > kScratchBytes)
    return fail(SF_ERR_WORKSPACE, "the no-allocation forward needs " + std::to_string(need) +
                                      " bytes of workspace; its static scratch holds " +
                                      std::to_string(kScratchBytes));
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != SF_OK) return s;
  return fwd_impl(shape, q, k, v, alpha, beta, S_in, o, S_out, nullptr, 0, ws, kScratchBytes,
                  stream, false);
}

static bool bad_phase(int phase) {
  if (phase == SF_PHASE_ALL || phase == SF_PHASE_BEGIN || phase == SF_PHASE_END) return false;
  fail(SF_ERR_INVALID_ARG, "phase must be SF_PHASE_ALL, SF_PHASE_BEGIN or SF_PHASE_END");
  return true;
}

sf_status sf_gdn_chunk_fwd_split(const sf_gdn_shape* shape, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const float* S_in, void* o, float* S_out, void* saved,
                                 size_t saved_bytes_, void* workspace, size_t ws_bytes, int phase,
                                 void* stream) {
  if (bad_phase(phase)) return SF_ERR_INVALID_ARG;
  return fwd_impl(shape, q, k, v, alpha, beta, S_in, o, S_out, saved, saved_bytes_, workspace,
                  ws_bytes, stream, saved != nullptr, phase);
}

sf_status sf_gdn_chunk_bwd_saved_split(const sf_gdn_shape* shape, const void* q, const void* k,
                                       const void* v, const float* alpha, const float* beta,
                                       const void* saved, size_t saved_bytes_, const void* dO,
                                       const float* dS_out, void* dq, void* dk, void* dv,
                                       float* dalpha, float* dbeta, float* dS_in, void* workspace,
                                       size_t ws_bytes, int phase, void* stream) {
  if (bad_phase(phase)) return SF_ERR_INVALID_ARG;
  return bwd_impl(shape, q, k, v, alpha, beta, nullptr, saved, saved_bytes_, dO, dS_out, dq, dk,
                  dv, dalpha, dbeta, dS_in, workspace, ws_bytes, stream, true, phase);
}

const char* sf_status_string(int status) {
  switch (status) {
    case SF_OK: return "SF_OK";
    case SF_ERR_INVALID_ARG: return "SF_ERR_INVALID_ARG";
    case SF_ERR_UNSUPPORTED: return "SF_ERR_UNSUPPORTED";
    case SF_ERR_WORKSPACE: return "SF_ERR_WORKSPACE";
    case SF_ERR_HIP: return "SF_ERR_HIP";
    default: return "SF_ERR_UNKNOWN";
  }
}

const char* sf_last_error_message(void) { return g_err.c_str(); }

const char* sf_gdn_version(void) { return "sf_gdn 0.1 (gfx950)"; }

sf_status sf_gdn_profile_begin(int capacity) {
  if (capacity <= 0) return fail(SF_ERR_INVALID_ARG, "capacity must be positive");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.recs.clear();
  g_prof.names.clear();
  g_prof.counts.clear();
  g_prof.ms.clear();
  g_prof.ev.resize((size_t)capacity * 2);
  for (auto& e : g_prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      g_prof.ev.clear();
      return hip_fail(r, "hipEventCreate");
    }
  }
  g_prof.on.store(true, std::memory_order_release);
  return SF_OK;
}

sf_status sf_gdn_profile_end(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on.store(false, std::memory_order_release);
  for (const ProfRec& r : g_prof.recs) {
    hipError_t e = hipEventSynchronize(g_prof.ev[r.ev + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float t = 0.f;
    e = hipEventElapsedTime(&t, g_prof.ev[r.ev], g_prof.ev[r.ev + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    size_t i = 0;
    while (i < g_prof.names.size() && g_prof.names[i] != r.name) ++i;
    if (i == g_prof.names.size()) {
      g_prof.names.push_back(r.name);
      g_prof.counts.push_back(0);
      g_prof.ms.push_back(0.0);
    }
    g_prof.counts[i] += 1;
    g_prof.ms[i] += t;
  }
  g_prof.recs.clear();
  return SF_OK;
}

int sf_gdn_profile_kernel_count(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  return (int)g_prof.names.size();
}

sf_status sf_gdn_profile_kernel(int index, const char** name, long long* launches,
                                double* total_ms) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (index < 0 || index >= (int)g_prof.names.size())
    return fail(SF_ERR_INVALID_ARG, "profile index out of range");
  if (name) *name = g_prof.names[index].c_str();
  if (launches) *launches = g_prof.counts[index];
  if (total_ms) *total_ms = g_prof.ms[index];
  return SF_OK;
}


sf_status sf_gdn_shortconv_fwd(const sf_conv_shape* shape, const void* x, const float* w,
                               const void* conv_in, void* y, void* conv_out, void* stream) {
  ConvPlan p;
  sf_status s = make_conv_plan(shape, p);
  if (s != SF_OK) return s;
  const size_t es = p.dtype == SF_DTYPE_BF16 ? 2 : 4;
  const size_t ntok = (size_t)p.B * p.T * p.C * es, nst = (size_t)p.B * (p.W - 1) * p.C * es;
  if (!w) return fail(SF_ERR_INVALID_ARG, "w is required");
  if (p.T > 0 && (!x || !y)) return fail(SF_ERR_INVALID_ARG, "x and y are required");
  std::vector<Range> in = {{x, ntok, "x"}, {w, (size_t)p.C * p.W * 4, "w"}, {conv_in, nst, "conv_in"}};
  std::vector<Range> out = {{y, ntok, "y"}, {conv_out, nst, "conv_out"}};
  if ((s = check_ptrs(in, out, {})) != SF_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  return run_locked([&](Profiler* prof) -> sf_status {
    ConvArgs a{};
    a.x = x; a.w = w; a.cin = conv_in; a.y = y; a.cout = conv_out;
    a.B = p.B; a.T = p.T; a.C = p.C; a.W = p.W; a.act = p.act;
    hipError_t e = p.dtype == SF_DTYPE_BF16 ? launch_conv_fwd<bf16>(a, st, prof)
                                           : launch_conv_fwd<float>(a, st, prof);
    if (e != hipSuccess) return hip_fail(e, "convolution launch");
    return SF_OK;
  });
}

sf_status sf_gdn_shortconv_bwd_workspace_size(const sf_conv_shape* shape, size_t* bytes) {
  ConvPlan p;
  sf_status s = make_conv_plan(shape, p);
  if (s != SF_OK) return s;
  if (!bytes) return fail(SF_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = conv_bwd_ws(p);
  return SF_OK;
}

sf_status sf_gdn_shortconv_bwd(const sf_conv_shape* shape, const void* x, const float* w,
                               const void* conv_in, const void* dy, const void* dconv_out,
                               void* dx, float* dw, void* dconv_in, void* workspace,
                               size_t ws_bytes, void* stream) {
  ConvPlan p;
  sf_status s = make_conv_plan(shape, p);
  if (s != SF_OK) return s;
  const size_t es = p.dtype == SF_DTYPE_BF16 ? 2 : 4;
  const size_t ntok = (size_t)p.B * p.T * p.C * es, nst = (size_t)p.B * (p.W - 1) * p.C * es;
  if (!w || !dw) return fail(SF_ERR_INVALID_ARG, "w and dw are required");
  if (p.T > 0 && (!x || !dy || !dx)) return fail(SF_ERR_INVALID_ARG, "x, dy and dx are required");
  std::vector<Range> in = {{x, ntok, "x"}, {w, (size_t)p.C * p.W * 4, "w"}, {conv_in, nst, "conv_in"},
                           {dy, ntok, "dy"}, {dconv_out, nst, "dconv_out"},
                           {workspace, ws_bytes, "workspace"}};
  std::vector<Range> out = {{dx, ntok, "dx"}, {dw, (size_t)p.C * p.W * 4, "dw"},
                            {dconv_in, nst, "dconv_in"}};
  if ((s = check_ptrs(in, out, {})) != SF_OK) return s;
  const size_t need = conv_bwd_ws(p);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(SF_ERR_WORKSPACE, "convolution backward workspace needs " + std::to_string(need) + " bytes");
  if (workspace && ((uintptr_t)workspace % kAlign))
    return fail(SF_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  return run_locked([&](Profiler* prof) -> sf_status {
    ConvArgs a{};
    a.x = x; a.w = w; a.cin = conv_in; a.dy = dy; a.dcout = dconv_out;
    a.dx = dx; a.dw = dw; a.dcin = dconv_in;
    a.B = p.B; a.T = p.T; a.C = p.C; a.W = p.W; a.act = p.act;
    hipError_t e = p.dtype == SF_DTYPE_BF16
                       ? launch_conv_bwd<bf16>(a, p.GR, (float*)workspace, st, prof)
                       : launch_conv_bwd<float>(a, p.GR, (float*)workspace, st, prof);
    if (e != hipSuccess) return hip_fail(e, "convolution launch");
    return SF_OK;
  });
}

}  // extern "C"
