// Per-block pieces of the chunkwise (WY/UT) gated delta rule.
//
// For one block of C = 64 tokens with block-local log-decay g_r =
// sum_{j<=r} log alpha_j, Gamma_rs = exp(g_r - g_s) (s <= r), gamma = e^g and
// D_r = exp(g_C - g_r), the token recurrence of the gated delta rule (Gated
// DeltaNet; the page's Eq. (1) and its "V_new" path of Eq. (2), Pith review of
// StateFlow, Referee Report, major comment 1) is equivalent to
//
//   A   = strict lower part of diag(beta) (K K^T o Gamma)
//   T   = (I + A)^{-1}
//   W   = T diag(beta o gamma) K,      U = T diag(beta) V
//   Vn  = U - W S^T                    (the effective values written)
//   O   = diag(gamma) Q S^T + (lower part incl. diagonal of Q K^T o Gamma) Vn
//   S'  = gamma_C S + Vn^T D K
//
// This is the "Pre / ST / Out" split the page describes (Figure 2 caption):
// A, T, W, U are state independent (Pre), Vn and S' carry the state (ST), O
// is the output (Out).  Reading of the page: no query scale, scalar gates
// per token and head, decay multiplies the whole previous state.
#pragma once
#include "gdn_device.hpp"

namespace sfgdn {

// Block gate vectors in LDS.
struct GateLds {
  float* g;     // block-local inclusive cumsum of log alpha
  float* gam;   // exp(g)
  float* beta;  // beta
  float* bg;    // beta * exp(g)
  float* dec;   // exp(g_C - g)
  float* gC;    // [0] = exp(g_C), [1] = g_C
};
constexpr size_t kGateBytes = 6 * BLK * sizeof(float) + 16;

__device__ __forceinline__ GateLds gate_lds(unsigned char* base) {
  float* f = reinterpret_cast<float*>(base);
  return GateLds{f, f + BLK, f + 2 * BLK, f + 3 * BLK, f + 4 * BLK, f + 5 * BLK};
}

// Wave 0 only: lane r holds log(alpha_r) and beta_r of token r (0 and 0 for
// rows past the end of the sequence, which then leave the state unchanged).
__device__ __forceinline__ void block_gates(float la, float be, const GateLds& G) {
  const int lane = lane_id();
  const float x = wave_prefix_sum(la);
  const float gC = lane_f(x, 63);
  const float gm = __expf(x);
  G.g[lane] = x;
  G.gam[lane] = gm;
  G.beta[lane] = be;
  G.bg[lane] = be * gm;
  G.dec[lane] = __expf(gC - x);
  if (lane == 0) {
    G.gC[0] = __expf(gC);
    G.gC[1] = gC;
  }
}

// Scores of an NW-wave workgroup (NW = 4 or 8): wave w owns s-tile w % 4 and
// r-tiles from (w / 4) * (16 / NW).
//   Af[r][s] = (s < r) beta_r Gamma_rs k_r.k_s      (fp32, strictly lower), if WITH_A
//   Pl[r][s] = (s <= r) Gamma_rs q_r.k_s            (operand type), if WITH_Q
// Computed as K K^T and K Q^T with s on the accumulator's m index so each
// lane stores 4 consecutive s.  A_OVER_K: Af lies over the K tile (a barrier
// separates the last K read from the first A write).
template <typename T, int D, int NW, bool WITH_Q, bool WITH_A = true, bool A_OVER_K = false>
__device__ __forceinline__ void block_scores(const T* Qs, const T* Ks, int ldd, const GateLds& G,
                                             float* Af, int ldf, T* Pl, int ldc,
                                             f32x4* kk = nullptr) {
  constexpr int NJ = 16 / NW;
  const int w = wave_id(), lane = lane_id();
  const int st = w & 3, r0 = (w >> 2) * NJ;
  f32x4 accA[NJ], accP[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) accA[j] = accP[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
    const auto a = frag_row<T, STD>(Ks + 16 * st * ldd, ldd, s);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (WITH_A)
        accA[j] = Mma<T>::mma(a, frag_row<T, STD>(Ks + 16 * (r0 + j) * ldd, ldd, s), accA[j]);
      if constexpr (WITH_Q)
        accP[j] = Mma<T>::mma(a, frag_row<T, STD>(Qs + 16 * (r0 + j) * ldd, ldd, s), accP[j]);
    }
  }
  // Af takes the K tile's region: every wave's K reads end before any A write
  if constexpr (A_OVER_K) lds_barrier();
  if (kk) {  // the raw K K^T tiles (m = st, n = r0 + j), for callers that need them later
#pragma unroll
    for (int j = 0; j < NJ; ++j) kk[j] = accA[j];
  }
  const int s0 = 16 * st + 4 * (lane >> 4);
  float gs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) gs[e] = G.g[s0 + e];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = 16 * (r0 + j) + (lane & 15);
    const float gr = G.g[r], br = G.beta[r];
    float a[4], p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = s0 + e;
      const float gam = (s <= r) ? __expf(gr - gs[e]) : 0.f;
      a[e] = (s < r) ? br * gam * accA[j][e] : 0.f;
      p[e] = gam * accP[j][e];
    }
    if constexpr (WITH_A) st4(Af + r * ldf + s0, a[0], a[1], a[2], a[3]);
    if constexpr (WITH_Q) st4(lds_sw(Pl + r * ldc + s0, ldc), p[0], p[1], p[2], p[3]);
  }
}

// T = (I + A)^{-1} for the strictly lower 64x64 A, in fp32 (needs >= 4 waves).
// The four 16x16 diagonal blocks are solved by forward substitution (one lane
// per column); the off-diagonal blocks follow by block recursion on MFMA,
//   T_ij = -T_ii (sum_k A_ik T_kj),
// first for the pairs (1,0) and (3,2), then for rows 32..63 x cols 0..31.
// The upper blocks of Tm are never part of T; they serve as scratch here and
// must be treated as zero by readers.  Ends with a workgroup barrier.
// Tm may be Af (T over A in place): each block of A is read by the wave that
// then writes the block of T in its place, or before a barrier that precedes
// that write, and the scratch lies in the upper blocks, which A leaves unused.
// Wave SUBW does the substitution while the other waves run side(), work of
// their own that needs neither A nor T; wave SUBW runs its side() during the
// first block step, which occupies waves 0 and 1 only (SUBW >= 2 then).
struct NoSide {
  __device__ void operator()() const {}
};
template <int SUBW = 0, class Side = NoSide>
__device__ __forceinline__ void block_solve(const float* Af, float* Tm, int ldf,
                                            Side&& side = Side()) {
  static_assert(SUBW == 0 || SUBW >= 2, "the substituting wave runs its side work in step 1");
  const int w = wave_id(), lane = lane_id();
  if (w != SUBW) side();
  if (w == SUBW) {
    // the substitution is the workgroup's critical path here: its wave goes
    // ahead of the side work of the wave it shares a SIMD with
    __builtin_amdgcn_s_setprio(2);
    const int base = 16 * (lane >> 4), c = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) v -= Af[(base + r) * ldf + base + s] * x[s];
      x[r] = v;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[(base + r) * ldf + base + c] = x[r];
    __builtin_amdgcn_s_setprio(0);
  }
  lds_barrier();
  float* X = Tm + 16;  // blocks (0,1) and (0,2) as scratch: X_w at column 16 (w + 1)
  if (w < 2) {
    // X_w is written and read back by this wave alone: LDS operations of one
    // wave take effect in order, so no workgroup barrier sits between.
    const int ib = 2 * w + 1, jb = 2 * w;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    gemm_nn_f32<16>(acc, Af + 16 * ib * ldf + 16 * jb, ldf, Tm + 16 * jb * ldf + 16 * jb, ldf);
    store_tile_N(acc, X + 16 * w, ldf, 0, 0);
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    gemm_nn_f32<16>(acc, Tm + 16 * ib * ldf + 16 * ib, ldf, X + 16 * w, ldf);
    store_tile_N(acc, Tm + 16 * ib * ldf + 16 * jb, ldf, 0, 0, -1.f);
  }
  if (SUBW != 0 && w == SUBW) side();
  lds_barrier();
  float* R = Tm + 32;  // rows 0..31 x cols 32..63 (upper blocks) as scratch
  if (w < 4) {
    const int ib = 2 + (w >> 1), jb = w & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (jb == 0)  // A_{ib,0} T_{0,0} + A_{ib,1} T_{1,0}
      gemm_nn_f32<32>(acc, Af + 16 * ib * ldf, ldf, Tm, ldf);
    else          // A_{ib,1} T_{1,1}
      gemm_nn_f32<16>(acc, Af + 16 * ib * ldf + 16, ldf, Tm + 16 * ldf + 16, ldf);
    store_tile_N(acc, R + 16 * (ib - 2) * ldf + 16 * jb, ldf, 0, 0);
  }
  lds_barrier();
  if (w < 4) {
    const int ib = 2 + (w >> 1), jb = w & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (ib == 2)  // T_22 R_{2,jb}
      gemm_nn_f32<16>(acc, Tm + 32 * ldf + 32, ldf, R + 16 * jb, ldf);
    else          // T_32 R_{2,jb} + T_33 R_{3,jb}
      gemm_nn_f32<32>(acc, Tm + 48 * ldf + 32, ldf, R + 16 * jb, ldf);
    store_tile_N(acc, Tm + 16 * ib * ldf + 16 * jb, ldf, 0, 0, -1.f);
  }
  lds_barrier();
}

// Tp = T diag(beta o gamma) (unless Tp is null) and Tpp = T diag(beta), in the
// operand type, by a workgroup of NT threads, into LDS tiles (LDS_DST) or a
// plain row-major array in global memory.  Upper 16x16 blocks are written as
// zero.
template <typename T, int NT, bool LDS_DST>
__device__ __forceinline__ void block_tprime(const float* Tm, int ldf, const GateLds& G, T* Tp,
                                             T* Tpp, int ldc) {
  constexpr int EPT = BLK * BLK / NT;   // elements per thread
  constexpr int TPR = BLK / EPT;        // threads per row
  static_assert(EPT % 4 == 0 && EPT <= 16, "tprime split");
  const int r = threadIdx.x / TPR, s0 = (threadIdx.x % TPR) * EPT;
#pragma unroll
  for (int x = 0; x < EPT; x += 4) {
    const int s = s0 + x;
    const bool upper = (s >> 4) > (r >> 4);
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = upper ? 0.f : Tm[r * ldf + s + e];
    T* dp = Tp + r * ldc + s;
    T* dpp = Tpp + r * ldc + s;
    if constexpr (LDS_DST) {
      dp = lds_sw(dp, ldc);
      dpp = lds_sw(dpp, ldc);
    }
    if (Tp)
      st4(dp, t[0] * G.bg[s], t[1] * G.bg[s + 1], t[2] * G.bg[s + 2], t[3] * G.bg[s + 3]);
    st4(dpp, t[0] * G.beta[s], t[1] * G.beta[s + 1], t[2] * G.beta[s + 2],
        t[3] * G.beta[s + 3]);
  }
}

// The transpose read of rows k of a row-major tile (B operand over k, STD
// order) with element k scaled by gam[k].
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_tr_gamma(const T* p, int ld, int s,
                                                               const float* gam);
template <>
__device__ __forceinline__ bf16x8 frag_tr_gamma<bf16>(const bf16* p, int ld, int s,
                                                      const float* gam) {
  bf16x8 f = frag_tr<bf16, STD>(p, ld, s);
  const int r0 = 32 * s + 8 * (lane_id() >> 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)((float)f[j] * gam[r0 + j]);
  return f;
}
template <>
__device__ __forceinline__ float frag_tr_gamma<float>(const float* p, int ld, int s,
                                                      const float* gam) {
  return frag_tr<float, STD>(p, ld, s) * gam[4 * s + (lane_id() >> 4)];
}

// Wn = -W, row-major [r][dk], by a workgroup of NW waves (wave w: dk-tiles
// NDK*w ..): computed as W^T = K^T Tp^T with K^T read through the transpose
// read from the row-major K tile.  With gam, the tile given is Tpp = T
// diag(beta) and Tp = Tpp diag(gamma) is applied through K instead:
// W = Tpp (diag(gamma) K), each K^T operand element k scaled by gamma_k.
template <typename T, int D, int NW>
__device__ __forceinline__ void block_w(const T* Ks, int ldd, const T* Tp, int ldc, T* Wn,
                                        const float* gam = nullptr) {
  constexpr int NDK = D / 16 / NW;
  const int w = wave_id();
  f32x4 acc[NDK][4];
  zero_acc(acc);
#pragma unroll
  for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
    typename Mma<T>::frag bt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bt[j] = frag_row<T, STD>(Tp + 16 * j * ldc, ldc, s);
#pragma unroll
    for (int i = 0; i < NDK; ++i) {
      const auto a = gam ? frag_tr_gamma<T>(Ks + 16 * (NDK * w + i), ldd, s, gam)
                         : frag_tr<T, STD>(Ks + 16 * (NDK * w + i), ldd, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::mma(a, bt[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < NDK; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) store_tile_T(acc[i][j], Wn, ldd, 16 * (NDK * w + i), 16 * j, -1.f);
}

// U[s][dv] = (Tpp V)[s][dv] for this wave's dv-tiles dv0 .. dv0+NDV-1, into
// register tiles u[dv-tile][s-tile] (s on the accumulator's m index).
template <typename T, int NDV>
__device__ __forceinline__ void block_u(const T* Tpp, int ldc, const T* Vs, int ldd, int dv0,
                                        f32x4 (&u)[NDV][4]) {
#pragma unroll
  for (int b = 0; b < NDV; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) u[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
    typename Mma<T>::frag bv[NDV];
#pragma unroll
    for (int b = 0; b < NDV; ++b) bv[b] = frag_tr<T, STD>(Vs + 16 * (dv0 + b), ldd, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto a = frag_row<T, STD>(Tpp + 16 * i * ldc, ldc, s);
#pragma unroll
      for (int b = 0; b < NDV; ++b) u[b][i] = Mma<T>::mma(a, bv[b], u[b][i]);
    }
  }
}

// acc[b][i] (m = s-tile i, n = dv-tile b) += X[s][:] . St[b]^T where the state
// tiles St[b][a] hold S^T (m = dk-tile a, n = dv-tile b) in registers; X is a
// row-major [s][dk] LDS tile (here -W).  Gives Vn = U - W S^T.
// PF: load the next k-step's operands before the current step's products
// (a scheduling barrier keeps the order), for kernels with registers to spare.
template <typename T, int D, int NDV, bool PF = false>
__device__ __forceinline__ void block_x_st(const T* X, int ldd, const f32x4 (&St)[NDV][D / 16],
                                           f32x4 (&acc)[NDV][4]) {
  constexpr int KS = D / Mma<T>::KSTEP;
  if constexpr (PF) {
    typename Mma<T>::frag a[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = frag_row<T, PERM>(X + 16 * i * ldd, ldd, 0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[(s + 1) & 1][i] = frag_row<T, PERM>(X + 16 * i * ldd, ldd, s + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      typename Mma<T>::frag bs[NDV];
#pragma unroll
      for (int b = 0; b < NDV; ++b) bs[b] = AccFrag<T>::get(St[b], s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < NDV; ++b) acc[b][i] = Mma<T>::mma(a[s & 1][i], bs[b], acc[b][i]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      typename Mma<T>::frag bs[NDV];
#pragma unroll
      for (int b = 0; b < NDV; ++b) bs[b] = AccFrag<T>::get(St[b], s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto a = frag_row<T, PERM>(X + 16 * i * ldd, ldd, s);
#pragma unroll
        for (int b = 0; b < NDV; ++b) acc[b][i] = Mma<T>::mma(a, bs[b], acc[b][i]);
      }
    }
  }
}

// block_x_st with the first NPF k-steps' X fragments read beforehand.
template <typename T, int D, int NDV, int NPF>
__device__ __forceinline__ void block_x_st_ra(const T* X, int ldd, const f32x4 (&St)[NDV][D / 16],
                                              const typename Mma<T>::frag (&a0)[NPF][4],
                                              f32x4 (&acc)[NDV][4]) {
  constexpr int KS = D / Mma<T>::KSTEP;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    typename Mma<T>::frag bs[NDV];
#pragma unroll
    for (int b = 0; b < NDV; ++b) bs[b] = AccFrag<T>::get(St[b], s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto a = s < NPF ? a0[s < NPF ? s : 0][i] : frag_row<T, PERM>(X + 16 * i * ldd, ldd, s);
#pragma unroll
      for (int b = 0; b < NDV; ++b) acc[b][i] = Mma<T>::mma(a, bs[b], acc[b][i]);
    }
  }
}

// acc[b][j] (m = dv-tile b, n = r-tile j) += S[dv][:] . Y[r][:] with S from the
// register state tiles and Y a row-major [r][dk] LDS tile (Q):  (S Y^T).
template <typename T, int D, int NDV>
__device__ __forceinline__ void block_s_yT(const f32x4 (&St)[NDV][D / 16], const T* Y, int ldd,
                                           f32x4 (&acc)[NDV][4]) {
#pragma unroll
  for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
    typename Mma<T>::frag bq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[j] = frag_row<T, PERM>(Y + 16 * j * ldd, ldd, s);
#pragma unroll
    for (int b = 0; b < NDV; ++b) {
      const auto a = AccFrag<T>::get(St[b], s);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[b][j] = Mma<T>::mma(a, bq[j], acc[b][j]);
    }
  }
}

// z[b][i] (m = s-tile i, n = dv-tile b) += K[s][:] . S[dv][:] and
// o[b][j] (m = dv-tile b, n = r-tile j) += S[dv][:] . Q[r][:], the state's
// operand fragments shared by both products.
template <typename T, int D, int NDV, bool WITH_Q = true>
__device__ __forceinline__ void block_s_kq(const f32x4 (&St)[NDV][D / 16], const T* Ks,
                                           const T* Qs, int ldd, f32x4 (&z)[NDV][4],
                                           f32x4 (&o)[NDV][4]) {
#pragma unroll
  for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
    typename Mma<T>::frag fk[4], fq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fk[i] = frag_row<T, PERM>(Ks + 16 * i * ldd, ldd, s);
      if constexpr (WITH_Q) fq[i] = frag_row<T, PERM>(Qs + 16 * i * ldd, ldd, s);
    }
#pragma unroll
    for (int b = 0; b < NDV; ++b) {
      const auto bs = AccFrag<T>::get(St[b], s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[b][i] = Mma<T>::mma(fk[i], bs, z[b][i]);
        if constexpr (WITH_Q) o[b][i] = Mma<T>::mma(bs, fq[i], o[b][i]);
      }
    }
  }
}

// Element (m = 4g + e, n = i) of the 16 x 16 tile at rows r0.., columns c0..
// of a row-major LDS tile, in an accumulator's lane layout.
template <typename T>
__device__ __forceinline__ f32x4 tile_acc_layout(const T* p, int ld, int r0, int c0);
template <>
__device__ __forceinline__ f32x4 tile_acc_layout<bf16>(const bf16* p, int ld, int r0, int c0) {
  const bf16x4 x = tr_rows4(p + c0, ld, r0 + 4 * (lane_id() >> 4));
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <>
__device__ __forceinline__ f32x4 tile_acc_layout<float>(const float* p, int ld, int r0, int c0) {
  const int l = lane_id(), m = r0 + 4 * (l >> 4), n = c0 + (l & 15);
  return f32x4{p[m * ld + n], p[(m + 1) * ld + n], p[(m + 2) * ld + n], p[(m + 3) * ld + n]};
}

// Vn = Tpp (V - diag(gamma) Z) for this wave's dv-tiles, Z = K S^T from
// block_s_kq (m = s, n = dv): X = V - gamma Z in registers, then the product
// with Tpp rows read in the accumulators' k order.
template <typename T, int NDV>
__device__ __forceinline__ void block_vn_from_z(const T* Tpp, int ldc, const T* Vs, int ldd,
                                                int dv0, const float* gam, f32x4 (&z)[NDV][4],
                                                f32x4 (&vn)[NDV][4]) {
  const int g4 = 4 * (lane_id() >> 4);
#pragma unroll
  for (int b = 0; b < NDV; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = tile_acc_layout<T>(Vs, ldd, 16 * i, 16 * (dv0 + b));
#pragma unroll
      for (int e = 0; e < 4; ++e) z[b][i][e] = v[e] - gam[16 * i + g4 + e] * z[b][i][e];
      vn[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
    typename Mma<T>::frag bx[NDV];
#pragma unroll
    for (int b = 0; b < NDV; ++b) bx[b] = AccFrag<T>::get(z[b], s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto a = frag_row<T, PERM>(Tpp + 16 * i * ldc, ldc, s);
#pragma unroll
      for (int b = 0; b < NDV; ++b) vn[b][i] = Mma<T>::mma(a, bx[b], vn[b][i]);
    }
  }
}

// acc[b][j] (m = dv-tile b, n = r-tile j) += Vn^T[dv][:] . P[r][:] with Vn in
// register tiles vn[b][s-tile] and P a row-major [r][s] LDS tile.
template <typename T, int NDV, bool PF = false>
__device__ __forceinline__ void block_vnT_pT(const f32x4 (&vn)[NDV][4], const T* Pl, int ldc,
                                             f32x4 (&acc)[NDV][4]) {
  constexpr int KS = BLK / Mma<T>::KSTEP;
  typename Mma<T>::frag bp[KS][4];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bp[s][j] = frag_row<T, PERM>(Pl + 16 * j * ldc, ldc, s);
    if constexpr (!PF) {
#pragma unroll
      for (int b = 0; b < NDV; ++b) {
        const auto a = AccFrag<T>::get(vn[b], s);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[b][j] = Mma<T>::mma(a, bp[s][j], acc[b][j]);
      }
    }
  }
  if constexpr (PF) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int b = 0; b < NDV; ++b) {
        const auto a = AccFrag<T>::get(vn[b], s);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[b][j] = Mma<T>::mma(a, bp[s][j], acc[b][j]);
      }
  }
}

// St[b][a] (m = dk-tile a, n = dv-tile b) += K^T[dk][:] . (D Vn)^T[dv][:]:
// the state update's write term Vn^T D K, with K^T through the transpose read
// from the row-major K tile and D Vn from the register tiles vn scaled by dsc.
template <typename T, int D, int NDV, bool PF = false>
__device__ __forceinline__ void block_state_write(const T* Ks, int ldd, const f32x4 (&vn)[NDV][4],
                                                  const f32x4 (&dsc)[4],
                                                  f32x4 (&St)[NDV][D / 16]) {
  constexpr int KS = BLK / Mma<T>::KSTEP, NA = D / 16, HA = NA / 2;
  if constexpr (PF) {
    // K^T operands in two halves of the dk-tiles, the next half loading while
    // the current one multiplies
    typename Mma<T>::frag ka[2][HA];
#pragma unroll
    for (int a = 0; a < HA; ++a) ka[0][a] = frag_tr<T, PERM>(Ks + 16 * a, ldd, 0);
#pragma unroll
    for (int st = 0; st < 2 * KS; ++st) {
      const int s = st >> 1, half = st & 1;
      if (st + 1 < 2 * KS) {
        const int s1 = (st + 1) >> 1, h1 = (st + 1) & 1;
#pragma unroll
        for (int a = 0; a < HA; ++a)
          ka[(st + 1) & 1][a] = frag_tr<T, PERM>(Ks + 16 * (h1 * HA + a), ldd, s1);
      }
      __builtin_amdgcn_sched_barrier(0);
      typename Mma<T>::frag bv[NDV];
#pragma unroll
      for (int b = 0; b < NDV; ++b) bv[b] = AccFrag<T>::get_scaled(vn[b], dsc, s);
#pragma unroll
      for (int a = 0; a < HA; ++a)
#pragma unroll
        for (int b = 0; b < NDV; ++b)
          St[b][half * HA + a] = Mma<T>::mma(ka[st & 1][a], bv[b], St[b][half * HA + a]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      typename Mma<T>::frag bv[NDV];
#pragma unroll
      for (int b = 0; b < NDV; ++b) bv[b] = AccFrag<T>::get_scaled(vn[b], dsc, s);
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const auto ka = frag_tr<T, PERM>(Ks + 16 * a, ldd, s);
#pragma unroll
        for (int b = 0; b < NDV; ++b) St[b][a] = Mma<T>::mma(ka, bv[b], St[b][a]);
      }
    }
  }
}

}  // namespace sfgdn
