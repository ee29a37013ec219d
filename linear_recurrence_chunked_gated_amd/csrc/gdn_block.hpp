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

// Distribution of a (16*TM) x (16*TN) tile grid over the workgroup's waves:
// each wave owns one 16-row m-tile and NJ consecutive n-tiles.
template <int TM, int TN> struct Dist {
  static constexpr int NJ = TM * TN / NWAVE;
  static_assert(TM <= NWAVE && (TM * TN) % NWAVE == 0 && NJ >= 1 && TN % NJ == 0,
                "tile grid does not split over the waves");
  __device__ static __forceinline__ int m(int w) { return w % TM; }
  __device__ static __forceinline__ int n0(int w) { return (w / TM) * NJ; }
};

// Block gate vectors in LDS.
struct GateLds {
  float* g;     // block-local inclusive cumsum of log alpha
  float* gam;   // exp(g)
  float* beta;  // beta
  float* bg;    // beta * exp(g)
  float* dec;   // exp(g_C - g)
  float* gC;    // [0] = exp(g_C), [1] = g_C
};

// Wave 0 only: lane r holds log(alpha_r) and beta_r of token r (0 and 0 for
// rows past the end of the sequence, which then leave the state unchanged).
__device__ __forceinline__ void block_gates(float la, float be, const GateLds& G) {
  const int lane = lane_id();
  float x = la;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  const float gC = __shfl(x, 63, 64);
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

// A (fp32, row-major, strictly lower) and, when WITH_Q, the masked decayed
// scores P[r][s] = (s <= r) Gamma_rs q_r.k_s (row-major, T).  Computed as
// transposed products (K K^T and K Q^T) so each lane stores 4 consecutive s.
template <typename T, int D, bool WITH_Q>
__device__ __forceinline__ void block_scores(const T* Qs, const T* Ks, int ldd, const GateLds& G,
                                             float* Af, int ldf, T* Pl, int ldc) {
  typedef Dist<4, 4> DS;
  const int w = wave_id(), lane = lane_id();
  const int mt = DS::m(w), nt0 = DS::n0(w);
  f32x4 accA[1][DS::NJ], accP[1][DS::NJ];
  zero_acc(accA);
  gemm_nt<T, 1, DS::NJ, D>(accA, Ks + 16 * mt * ldd, ldd, Ks + 16 * nt0 * ldd, ldd);
  if (WITH_Q) {
    zero_acc(accP);
    gemm_nt<T, 1, DS::NJ, D>(accP, Ks + 16 * mt * ldd, ldd, Qs + 16 * nt0 * ldd, ldd);
  }
  const int s0 = 16 * mt + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < DS::NJ; ++j) {
    const int r = 16 * (nt0 + j) + (lane & 15);
    const float gr = G.g[r], br = G.beta[r];
    float a[4], p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = s0 + e;
      const float gam = (s <= r) ? __expf(gr - G.g[s]) : 0.f;
      a[e] = (s < r) ? br * gam * accA[0][j][e] : 0.f;
      p[e] = gam * accP[0][j][e];
    }
    st4(Af + r * ldf + s0, a[0], a[1], a[2], a[3]);
    if (WITH_Q) st4(Pl + r * ldc + s0, p[0], p[1], p[2], p[3]);
  }
}

// T = (I + A)^{-1} for the strictly lower 64x64 A, in fp32.  The four 16x16
// diagonal blocks are solved by forward substitution (one lane per column);
// the off-diagonal blocks follow by block recursion on MFMA:
//   T_ij = -T_ii (sum_k A_ik T_kj)
// first for the sub-diagonal pairs (1,0), (3,2), then for rows 32..63 x cols
// 0..31 at once.  Upper blocks of Tm are left unwritten (they are zero).
// scratch needs 2*16*20 + 32*36 floats.  Ends with a workgroup barrier.
__device__ __forceinline__ void block_solve(const float* Af, float* Tm, int ldf, float* scratch) {
  const int w = wave_id(), lane = lane_id();
  if (w == 0) {
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
  }
  __syncthreads();
  float* X = scratch;               // two 16 x 20 blocks
  float* R = scratch + 2 * 16 * 20; // 32 x 36
  if (w < 2) {
    const int ib = 2 * w + 1, jb = 2 * w;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    gemm_nn_f32<16>(acc, Af + 16 * ib * ldf + 16 * jb, ldf, Tm + 16 * jb * ldf + 16 * jb, ldf);
    store_tile_N(acc, X + w * 16 * 20, 20, 0, 0);
  }
  __syncthreads();
  if (w < 2) {
    const int ib = 2 * w + 1, jb = 2 * w;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    gemm_nn_f32<16>(acc, Tm + 16 * ib * ldf + 16 * ib, ldf, X + w * 16 * 20, 20);
    store_tile_N(acc, Tm + 16 * ib * ldf + 16 * jb, ldf, 0, 0, -1.f);
  }
  __syncthreads();
  if (w < 4) {
    const int ib = 2 + (w >> 1), jb = w & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (jb == 0)  // A_{ib,0} T_{0,0} + A_{ib,1} T_{1,0}
      gemm_nn_f32<32>(acc, Af + 16 * ib * ldf, ldf, Tm, ldf);
    else          // A_{ib,1} T_{1,1}
      gemm_nn_f32<16>(acc, Af + 16 * ib * ldf + 16, ldf, Tm + 16 * ldf + 16, ldf);
    store_tile_N(acc, R + (ib - 2) * 16 * 36 + 16 * jb, 36, 0, 0);
  }
  __syncthreads();
  if (w < 4) {
    const int ib = 2 + (w >> 1), jb = w & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (ib == 2)  // T_22 R_{2,jb}
      gemm_nn_f32<16>(acc, Tm + 32 * ldf + 32, ldf, R + 16 * jb, 36);
    else          // T_32 R_{2,jb} + T_33 R_{3,jb}
      gemm_nn_f32<32>(acc, Tm + 48 * ldf + 32, ldf, R + 16 * jb, 36);
    store_tile_N(acc, Tm + 16 * ib * ldf + 16 * jb, ldf, 0, 0, -1.f);
  }
  __syncthreads();
}

// Tp = T diag(beta o gamma), Tpp = T diag(beta), in the operand type.
template <typename T>
__device__ __forceinline__ void block_tprime(const float* Tm, int ldf, const GateLds& G, T* Tp,
                                             T* Tpp, int ldc) {
  const int r = threadIdx.x >> 3, s0 = (threadIdx.x & 7) * 8;
  const bool upper = (s0 >> 4) > (r >> 4);
#pragma unroll
  for (int x = 0; x < 8; x += 4) {
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = upper ? 0.f : Tm[r * ldf + s0 + x + e];
    const int s = s0 + x;
    st4(Tp + r * ldc + s, t[0] * G.bg[s], t[1] * G.bg[s + 1], t[2] * G.bg[s + 2],
        t[3] * G.bg[s + 3]);
    st4(Tpp + r * ldc + s, t[0] * G.beta[s], t[1] * G.beta[s + 1], t[2] * G.beta[s + 2],
        t[3] * G.beta[s + 3]);
  }
}

// Wn = -W (row-major [r][dk]) from W^T = K^T Tp^T, and the U accumulator
// accU[m = s][n = dv] = (Tpp V)[s][dv] for this wave's tiles.
template <typename T, int D>
__device__ __forceinline__ void block_wu(const T* KTs, const T* VTs, const T* Tp, const T* Tpp,
                                         int ldc, T* Wn, int ldd,
                                         f32x4 (&accU)[1][Dist<4, D / 16>::NJ]) {
  typedef Dist<D / 16, 4> DW;
  typedef Dist<4, D / 16> DU;
  const int w = wave_id();
  f32x4 accW[1][DW::NJ];
  zero_acc(accW);
  gemm_nt<T, 1, DW::NJ, BLK>(accW, KTs + 16 * DW::m(w) * ldc, ldc, Tp + 16 * DW::n0(w) * ldc, ldc);
#pragma unroll
  for (int j = 0; j < DW::NJ; ++j)
    store_tile_T(accW[0][j], Wn, ldd, 16 * DW::m(w), 16 * (DW::n0(w) + j), -1.f);
  zero_acc(accU);
  gemm_nt<T, 1, DU::NJ, BLK>(accU, Tpp + 16 * DU::m(w) * ldc, ldc, VTs + 16 * DU::n0(w) * ldc, ldc);
}

}  // namespace sfgdn
