// Short causal depthwise convolution of one pipeline chunk, with the chunk's
// boundary state (the last W-1 inputs of the previous chunk).
//
// Source: Pith review of StateFlow, "What carries the argument" (a chunk
// carries auxiliary local-convolution states across its boundary besides
// S^in/S^out) and "Referee Report", major comment 1 (these short-convolution
// boundary states must be reconstructed for the chunked backward to match
// full-sequence training).  The pages do not print the convolution; the
// reading implemented here is the usual causal depthwise 1-D convolution of
// width W along the tokens, per channel c:
//     xe = [conv_in (W-1 rows) ; x (T rows)]
//     z_t = sum_j w[c][j] xe[t + W-1 - j],   y_t = z_t  or  SiLU(z_t)
//     conv_out = the last W-1 rows of xe.
// The work is streaming (a few flops per element), so the kernels are laid
// out for HBM: each thread walks a run of tokens for a few adjacent channels
// with the W-1 previous inputs in registers, so every input is read once.
#include "gdn_kernels.hpp"

namespace sfgdn {

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }
// d/dz of z * sigmoid(z)
__device__ __forceinline__ float dsilu(float z) {
  const float s = 1.f / (1.f + __expf(-z));
  return s * (1.f + z * (1.f - s));
}

// Channel-vector loads/stores of V consecutive elements.
template <typename T, int V> struct __attribute__((aligned(sizeof(T) * V))) CVec {
  T v[V];
};
template <typename T, int V>
__device__ __forceinline__ void ld_vec(const T* p, float (&out)[V]) {
  const CVec<T, V> r = *reinterpret_cast<const CVec<T, V>*>(p);
#pragma unroll
  for (int i = 0; i < V; ++i) out[i] = to_f(r.v[i]);
}
template <typename T, int V>
__device__ __forceinline__ void st_vec(T* p, const float (&in)[V]) {
  CVec<T, V> r;
#pragma unroll
  for (int i = 0; i < V; ++i) r.v[i] = (T)in[i];
  *reinterpret_cast<CVec<T, V>*>(p) = r;
}

// xe row u (u < W-1: conv_in, else x row u - (W-1)) of channels c .. c+V-1.
template <typename T, int V, int W>
__device__ __forceinline__ void ld_xe(const T* x, const T* cin, int u, int C, int c,
                                      float (&out)[V]) {
  if (u >= W - 1) {
    ld_vec<T, V>(x + (size_t)(u - (W - 1)) * C + c, out);
  } else if (cin) {
    ld_vec<T, V>(cin + (size_t)u * C + c, out);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) out[i] = 0.f;
  }
}

// ------------------------------------------------------------------ forward
// Thread: V channels, a run of TR tokens.  Grid: (channel groups, token runs, B).
constexpr int CONV_THREADS = 256;
constexpr int CONV_TR = 64;

template <typename T, int W, int V>
__global__ __launch_bounds__(CONV_THREADS) void conv_fwd_kernel(ConvArgs a) {
  const int c = (blockIdx.x * CONV_THREADS + threadIdx.x) * V;
  if (c >= a.C) return;
  const int b = blockIdx.z, t0 = blockIdx.y * CONV_TR, t1 = min(a.T, t0 + CONV_TR);
  const T* __restrict__ x = reinterpret_cast<const T*>(a.x) + (size_t)b * a.T * a.C;
  const T* __restrict__ cin =
      a.cin ? reinterpret_cast<const T*>(a.cin) + (size_t)b * (W - 1) * a.C : nullptr;
  T* __restrict__ y = reinterpret_cast<T*>(a.y) + (size_t)b * a.T * a.C;
  float wt[W][V];
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int i = 0; i < V; ++i) wt[j][i] = a.w[(size_t)(c + i) * W + j];
  // win[j] = xe row (t + W-1 - j) for the current t, j = 1 .. W-1 (previous inputs)
  float win[W][V];
#pragma unroll
  for (int j = 1; j < W; ++j) ld_xe<T, V, W>(x, cin, t0 + W - 1 - j, a.C, c, win[j]);
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {
    ld_vec<T, V>(x + (size_t)t * a.C + c, win[0]);
    float z[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < W; ++j) s += wt[j][i] * win[j][i];
      z[i] = a.act ? silu(s) : s;
    }
    st_vec<T, V>(y + (size_t)t * a.C + c, z);
#pragma unroll
    for (int j = W - 1; j >= 1; --j)
#pragma unroll
      for (int i = 0; i < V; ++i) win[j][i] = win[j - 1][i];
  }
}

// conv_out = xe rows T .. T+W-2 (from conv_in when T < W-1).
template <typename T, int W, int V>
__global__ __launch_bounds__(CONV_THREADS) void conv_state_kernel(ConvArgs a) {
  const int c = (blockIdx.x * CONV_THREADS + threadIdx.x) * V;
  if (c >= a.C) return;
  const int b = blockIdx.z, m = blockIdx.y;
  const T* x = reinterpret_cast<const T*>(a.x) + (size_t)b * a.T * a.C;
  const T* cin = a.cin ? reinterpret_cast<const T*>(a.cin) + (size_t)b * (W - 1) * a.C : nullptr;
  float r[V];
  ld_xe<T, V, W>(x, cin, a.T + m, a.C, c, r);
  st_vec<T, V>(reinterpret_cast<T*>(a.cout) + ((size_t)b * (W - 1) + m) * a.C + c, r);
}

// ----------------------------------------------------------------- backward
// g_u = dy_u * act'(z_u).  Thread: V channels, a run of GR tokens walked
// backwards with two register windows, the inputs x[t-W+1 .. t] and the
// gradients g[t .. t+W-1]:
//   dx_t   = sum_j w[j] g[t+j]            (+ dconv_out[t+W-1-T] if t+W-1 >= T)
//   dw[j] += g_t xe[t+W-1-j]              (per-run partial, reduced later)
// Each x and dy row is read once (plus a W-1 row halo per run).
template <typename T, int W, int V>
__device__ __forceinline__ void conv_g(const ConvArgs& a, const T* dy, const float (&wt)[W][V],
                                       const float (&xz)[W][V], int t, int c, float (&g)[V]) {
  // xz[j] = xe row (t + W-1 - j), i.e. x_{t-j}
  ld_vec<T, V>(dy + (size_t)t * a.C + c, g);
  if (a.act) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < W; ++j) z += wt[j][i] * xz[j][i];
      g[i] *= dsilu(z);
    }
  }
}

template <typename T, int W, int V>
__global__ __launch_bounds__(CONV_THREADS) void conv_bwd_kernel(ConvArgs a, int GR, float* dwp) {
  const int c = (blockIdx.x * CONV_THREADS + threadIdx.x) * V;
  if (c >= a.C) return;
  const int b = blockIdx.z, r0 = blockIdx.y * GR, r1 = min(a.T, r0 + GR);
  const size_t TC = (size_t)a.T * a.C;
  const T* __restrict__ x = reinterpret_cast<const T*>(a.x) + b * TC;
  const T* __restrict__ cin =
      a.cin ? reinterpret_cast<const T*>(a.cin) + (size_t)b * (W - 1) * a.C : nullptr;
  const T* __restrict__ dy = reinterpret_cast<const T*>(a.dy) + b * TC;
  const T* __restrict__ dco =
      a.dcout ? reinterpret_cast<const T*>(a.dcout) + (size_t)b * (W - 1) * a.C : nullptr;
  T* __restrict__ dx = reinterpret_cast<T*>(a.dx) + b * TC;
  float wt[W][V], dw[W][V];
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      wt[j][i] = a.w[(size_t)(c + i) * W + j];
      dw[j][i] = 0.f;
    }
  // gw[j] = g_{t+j} for the current t (zero past T); xw[j] = x_{t-j}.
  float gw[W][V], xw[W][V];
  {
    // g of the W-1 tokens after the run, from their own input windows
    const int te = r1;  // first token after the run
#pragma unroll
    for (int jj = 1; jj < W; ++jj) {
      const int t = te + jj - 1;
      if (t < a.T) {
        float xz[W][V];
#pragma unroll
        for (int j = 0; j < W; ++j) ld_xe<T, V, W>(x, cin, t + W - 1 - j, a.C, c, xz[j]);
        conv_g<T, W, V>(a, dy, wt, xz, t, c, gw[jj]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) gw[jj][i] = 0.f;
      }
    }
    // inputs x_{r1-1-j}, j = 0 .. W-1 (the window of t = r1 - 1)
#pragma unroll
    for (int j = 0; j < W; ++j) ld_xe<T, V, W>(x, cin, r1 - 1 + W - 1 - j, a.C, c, xw[j]);
  }
  // One token t (walking down): g_t, dx_t, this token's dw terms, then the
  // windows move down and take x_{t-W} (xe row t-1).  TAIL: t + W-1 >= T, so
  // dx_t also takes dconv_out[t+W-1-T]; HEAD: xe row t-1 may lie in conv_in.
  auto token = [&](int t, bool tail, bool head) {
    float g0[V];
    conv_g<T, W, V>(a, dy, wt, xw, t, c, g0);
#pragma unroll
    for (int i = 0; i < V; ++i) gw[0][i] = g0[i];
    float o[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < W; ++j) s += wt[j][i] * gw[j][i];
      o[i] = s;
#pragma unroll
      for (int j = 0; j < W; ++j) dw[j][i] += gw[0][i] * xw[j][i];
    }
    if (tail && dco) {
      float e[V];
      ld_vec<T, V>(dco + (size_t)(t + W - 1 - a.T) * a.C + c, e);
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] += e[i];
    }
    st_vec<T, V>(dx + (size_t)t * a.C + c, o);
#pragma unroll
    for (int j = W - 1; j >= 1; --j)
#pragma unroll
      for (int i = 0; i < V; ++i) gw[j][i] = gw[j - 1][i];
#pragma unroll
    for (int j = 0; j + 1 < W; ++j)
#pragma unroll
      for (int i = 0; i < V; ++i) xw[j][i] = xw[j + 1][i];
    if (head) {
      if (t - 1 >= r0) ld_xe<T, V, W>(x, cin, t - 1, a.C, c, xw[W - 1]);
    } else {
      ld_vec<T, V>(x + (size_t)(t - W) * a.C + c, xw[W - 1]);  // t >= W: a plain x row
    }
  };
  // The last W-1 tokens of the sequence (dconv_out term), then the bulk with
  // plain x rows and no branches, then the first W tokens (conv_in rows).
  int t = r1 - 1;
  for (; t >= r0 && t > a.T - W; --t) token(t, true, t < W);
  const int tlo = max(r0, W);
#pragma unroll 8
  for (; t >= tlo; --t) token(t, false, false);
  for (; t >= r0; --t) token(t, false, true);
  // this run's dw partial: dwp[(b * nrun + run)][c][j]
  const int nrun = gridDim.y;
  float* p = dwp + ((size_t)b * nrun + blockIdx.y) * a.C * W;
#pragma unroll
  for (int i = 0; i < V; ++i)
#pragma unroll
    for (int j = 0; j < W; ++j) p[(size_t)(c + i) * W + j] = dw[j][i];
}

// dconv_in[m] = sum_j w[j] g[m-(W-1)+j] (+ dconv_out[m-T] if m >= T).  One
// thread per (b, m, channel group); g recomputed from dy (and x for SiLU).
template <typename T, int W, int V>
__global__ __launch_bounds__(CONV_THREADS) void conv_dstate_kernel(ConvArgs a) {
  const int c = (blockIdx.x * CONV_THREADS + threadIdx.x) * V;
  if (c >= a.C) return;
  const int b = blockIdx.z, m = blockIdx.y;
  const size_t TC = (size_t)a.T * a.C;
  const T* x = reinterpret_cast<const T*>(a.x) + b * TC;
  const T* cin = a.cin ? reinterpret_cast<const T*>(a.cin) + (size_t)b * (W - 1) * a.C : nullptr;
  const T* dy = reinterpret_cast<const T*>(a.dy) + b * TC;
  float o[V];
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] = 0.f;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const int t = m - (W - 1) + j;
    if (t < 0 || t >= a.T) continue;
    float d[V];
    ld_vec<T, V>(dy + (size_t)t * a.C + c, d);
    if (a.act) {
      float xe[W][V];
#pragma unroll
      for (int jj = 0; jj < W; ++jj) ld_xe<T, V, W>(x, cin, t + W - 1 - jj, a.C, c, xe[jj]);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float z = 0.f;
#pragma unroll
        for (int jj = 0; jj < W; ++jj) z += a.w[(size_t)(c + i) * W + jj] * xe[jj][i];
        d[i] *= dsilu(z);
      }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) o[i] += a.w[(size_t)(c + i) * W + j] * d[i];
  }
  if (m >= a.T && a.dcout) {
    float e[V];
    ld_vec<T, V>(reinterpret_cast<const T*>(a.dcout) + ((size_t)b * (W - 1) + (m - a.T)) * a.C + c, e);
#pragma unroll
    for (int i = 0; i < V; ++i) o[i] += e[i];
  }
  st_vec<T, V>(reinterpret_cast<T*>(a.dcin) + ((size_t)b * (W - 1) + m) * a.C + c, o);
}

// out[g][i] = sum of parts g*grp .. min(nparts, (g+1)*grp) - 1 of src[p][i], in
// order.  Two passes (groups of CONV_GRP, then the group sums) give the weight
// gradient in a fixed order with enough parallelism.
constexpr int CONV_GRP = 32;
__global__ __launch_bounds__(CONV_THREADS) void conv_dw_reduce_kernel(const float* src, int nparts,
                                                                      int grp, int CW, float* out) {
  const int i = blockIdx.x * CONV_THREADS + threadIdx.x;
  if (i >= CW) return;
  const int p0 = blockIdx.y * grp, p1 = min(nparts, p0 + grp);
  float s = 0.f;
  for (int p = p0; p < p1; ++p) s += src[(size_t)p * CW + i];
  out[(size_t)blockIdx.y * CW + i] = s;
}

// ------------------------------------------------------------------ launch
template <typename T> constexpr int conv_vf() { return 16 / sizeof(T); }  // fwd channels/thread
template <typename T> constexpr int conv_vb() { return 8 / sizeof(T); }   // bwd channels/thread

template <typename T, int W>
static hipError_t conv_fwd_w(const ConvArgs& a, hipStream_t st, Profiler* prof) {
  constexpr int V = conv_vf<T>();
  const int gx = (a.C / V + CONV_THREADS - 1) / CONV_THREADS;
  if (a.T > 0) {
    prof_begin(prof, "conv_fwd", st);
    hipLaunchKernelGGL((conv_fwd_kernel<T, W, V>), dim3(gx, (a.T + CONV_TR - 1) / CONV_TR, a.B),
                       dim3(CONV_THREADS), 0, st, a);
    prof_end(prof, st);
  }
  if (W > 1 && a.cout) {
    prof_begin(prof, "conv_state", st);
    hipLaunchKernelGGL((conv_state_kernel<T, W, V>), dim3(gx, W - 1, a.B), dim3(CONV_THREADS), 0,
                       st, a);
    prof_end(prof, st);
  }
  return hipGetLastError();
}

template <typename T, int W>
static hipError_t conv_bwd_w(const ConvArgs& a, int GR, float* dwp, hipStream_t st,
                             Profiler* prof) {
  constexpr int V = conv_vb<T>();
  const int gx = (a.C / V + CONV_THREADS - 1) / CONV_THREADS;
  const int nrun = a.T > 0 ? (a.T + GR - 1) / GR : 0;
  if (a.T > 0) {
    prof_begin(prof, "conv_bwd", st);
    hipLaunchKernelGGL((conv_bwd_kernel<T, W, V>), dim3(gx, nrun, a.B), dim3(CONV_THREADS), 0, st,
                       a, GR, dwp);
    prof_end(prof, st);
    const int CW = a.C * W, np = a.B * nrun, ng = (np + CONV_GRP - 1) / CONV_GRP;
    const int bx = (CW + CONV_THREADS - 1) / CONV_THREADS;
    float* mid = dwp + (size_t)np * CW;  // ng group sums
    prof_begin(prof, "conv_dw_reduce", st);
    hipLaunchKernelGGL(conv_dw_reduce_kernel, dim3(bx, ng), dim3(CONV_THREADS), 0, st, dwp, np,
                       CONV_GRP, CW, mid);
    hipLaunchKernelGGL(conv_dw_reduce_kernel, dim3(bx, 1), dim3(CONV_THREADS), 0, st,
                       (const float*)mid, ng, ng, CW, a.dw);
    prof_end(prof, st);
  } else if (a.dw) {
    hipLaunchKernelGGL(conv_dw_reduce_kernel, dim3((a.C * W + CONV_THREADS - 1) / CONV_THREADS, 1),
                       dim3(CONV_THREADS), 0, st, dwp, 0, 1, a.C * W, a.dw);
  }
  if (W > 1 && a.dcin) {
    prof_begin(prof, "conv_dstate", st);
    hipLaunchKernelGGL((conv_dstate_kernel<T, W, V>), dim3(gx, W - 1, a.B), dim3(CONV_THREADS), 0,
                       st, a);
    prof_end(prof, st);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st, Profiler* prof) {
  switch (a.W) {
    case 1: return conv_fwd_w<T, 1>(a, st, prof);
    case 2: return conv_fwd_w<T, 2>(a, st, prof);
    case 3: return conv_fwd_w<T, 3>(a, st, prof);
    case 4: return conv_fwd_w<T, 4>(a, st, prof);
    case 5: return conv_fwd_w<T, 5>(a, st, prof);
    case 6: return conv_fwd_w<T, 6>(a, st, prof);
    case 7: return conv_fwd_w<T, 7>(a, st, prof);
    case 8: return conv_fwd_w<T, 8>(a, st, prof);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_conv_bwd(const ConvArgs& a, int GR, float* dwp, hipStream_t st, Profiler* prof) {
  switch (a.W) {
    case 1: return conv_bwd_w<T, 1>(a, GR, dwp, st, prof);
    case 2: return conv_bwd_w<T, 2>(a, GR, dwp, st, prof);
    case 3: return conv_bwd_w<T, 3>(a, GR, dwp, st, prof);
    case 4: return conv_bwd_w<T, 4>(a, GR, dwp, st, prof);
    case 5: return conv_bwd_w<T, 5>(a, GR, dwp, st, prof);
    case 6: return conv_bwd_w<T, 6>(a, GR, dwp, st, prof);
    case 7: return conv_bwd_w<T, 7>(a, GR, dwp, st, prof);
    case 8: return conv_bwd_w<T, 8>(a, GR, dwp, st, prof);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_conv_fwd<bf16>(const ConvArgs&, hipStream_t, Profiler*);
template hipError_t launch_conv_fwd<float>(const ConvArgs&, hipStream_t, Profiler*);
template hipError_t launch_conv_bwd<bf16>(const ConvArgs&, int, float*, hipStream_t, Profiler*);
template hipError_t launch_conv_bwd<float>(const ConvArgs&, int, float*, hipStream_t, Profiler*);

}  // namespace sfgdn
