// Backward kernels of one pipeline chunk of the gated delta rule.
//
// The chunk backward ("Bwd_i(Sbar_i^out) -> Sbar_i^in", Eq. 7 of the Pith
// review of StateFlow, "What carries the argument") rebuilds the chunk's state
// trajectory from its inputs (Referee Report, major comment 1: the backward
// must reconstruct the same intra-chunk trajectory, including V_new) and runs
// the state gradient backwards through it.  Per block, with dS' the gradient
// with respect to the block's exit state,
//   dVn = P^T dO + D K dS'^T
//   dS  = gamma_C dS' + dO^T diag(gamma) Q - dVn^T W     (entry-state gradient)
// which, like the forward, is affine: dS = dS' M_b^T + NB_b.  The launch
// sequence is
//   0. per-block Tp, Tpp                                  [forward Pre kernel]
//   1. segment maps (M, N) of the forward                       [forward kernel]
//   2. gdn_bwd_dscan<summary>: per segment, dS at its entry from a zero exit
//      gradient (NB_seg)
//   3. forward chain of entry states, reverse chain of exit gradients
//   4. block entry states h_b and V^new of every block             [forward kernel]
//   5. gdn_bwd_dscan<main>: per segment from its true exit gradient, the exit
//      gradient dS'_b of every block, and dS_in
//   6. gdn_bwd_grads: per block, fully parallel, dq dk dv dalpha dbeta.
#include <algorithm>

#include "gdn_kernels.hpp"

namespace sfgdn {

template <typename T, int D>
__device__ __forceinline__ const T* tok_base(const void* p, int T_, int H, int b, int h) {
  return reinterpret_cast<const T*>(p) + ((size_t)b * T_ * H + h) * D;
}

// ------------------------------------------------------------------ LDS ----
// dscan: RQ Q | RK K | RO dO | RW Wn | RT Tpp | RP P | RG gates.  Where that
// would not fit (fp32 operands at d = 128), Wn shares Q's region: the
// products that read Q then finish before W is formed, with a barrier between.
template <typename T, int D> struct ScanLds {
  static constexpr int LDD = D + Lay<T>::PAD;
  static constexpr int LDC = BLK + Lay<T>::PAD;
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t sq = (size_t)BLK * LDC * sizeof(T);
  static constexpr bool W_IN_Q = 4 * rowD + 2 * sq + kGateBytes > 160 * 1024;
  static constexpr size_t oQ = 0, oK = oQ + rowD, oO = oK + rowD, oW = W_IN_Q ? oQ : oO + rowD,
                          oT = (W_IN_Q ? oO : oW) + rowD, oP = oT + sq, oG = oP + sq;
  static constexpr size_t bytes = oG + kGateBytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(sizeof(T) != 2 || (oK % 4096 == 0 && oO % 4096 == 0 && oW % 4096 == 0 &&
                                   oT % 4096 == 0 && oP % 4096 == 0), "swizzled tiles 4 KiB aligned");
};

// Per-block inputs of the reverse scan in flight (q, k, dO rows, Tpp from the
// Pre kernel and gates).
template <typename T, int D> struct ScanPrefetch {
  typedef Tile<T, D, 4 * D> Tl;
  typedef Tile<T, BLK, 4 * D> Tt;
  uint4 rq[Tl::NCH], rk[Tl::NCH], ro[Tl::NCH], rp[Tt::NCH];
  float ra = 1.f, rb = 0.f;  // raw gates of the next block (wave 0)
  // PART: 1 the gates and Tpp, 2 q and k, 4 dO (bit mask); spread over a
  // block so that the address unit works beside the matrix work.
  template <int PART = 7>
  __device__ __forceinline__ void fetch(const T* q, const T* k, const T* dO, const float* al,
                                        const float* bt, const T* tp, size_t rs, int H, int t0,
                                        int nv) {
    if constexpr (PART & 1) {
      if (wave_id() == 0) {
        const size_t idx = (size_t)(t0 + min(lane_id(), nv - 1)) * H;
        ra = al[idx];
        rb = bt[idx];
      }
      Tt::load(rp, tp, BLK, BLK);
    }
    if constexpr (PART & 2) {
      Tl::load(rq, q + (size_t)t0 * rs, rs, nv);
      Tl::load(rk, k + (size_t)t0 * rs, rs, nv);
    }
    if constexpr (PART & 4) Tl::load(ro, dO + (size_t)t0 * rs, rs, nv);
  }
  __device__ __forceinline__ void stage(T* Qs, T* Ks, T* Os, T* Tp, int ld, int ldc, int nv,
                                        const GateLds& G) {
    Tt::to_lds(rp, Tp, ldc, BLK);
    Tl::to_lds(rq, Qs, ld, nv);
    Tl::to_lds(rk, Ks, ld, nv);
    Tl::to_lds(ro, Os, ld, nv);
    if (wave_id() == 0) {
      const bool ok = lane_id() < nv;
      block_gates(ok ? __logf(ra) : 0.f, ok ? rb : 0.f, G);
    }
  }
};

// Tpp = T diag(beta) of block blk of sequence bh ([64][64]; the Pre kernel
// stores only Tpp, Tp = Tpp diag(gamma) is applied through K).
template <typename T>
__device__ __forceinline__ const T* tp_block(const void* tw, int nblk, int bh, int blk) {
  return reinterpret_cast<const T*>(tw) + ((size_t)bh * nblk + blk) * BLK * BLK;
}

// ------------------------------------------------------- reverse dS scan ---
// Wave w owns dv-tile w of the state gradient dSv (tiles m = dk, n = dv, i.e.
// dS^T).  Blocks of the segment are visited last to first.  MAIN: start from
// the segment's exit gradient, store dS' of every block to dhst and dS_in from
// segment 0.  Otherwise: start from zero and store the segment's NB map.
template <typename T, int D, bool MAIN>
__global__ __launch_bounds__(4 * D, 2) void gdn_bwd_dscan_kernel(BwdArgs a, int seg0, int nseg,
                                                                 const float* dSend,
                                                                 int dsend_P) {
  typedef ScanLds<T, D> Lz;
  constexpr int DKT = D / 16, NW = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC;
  extern __shared__ __align__(16) unsigned char smem[];
  T* Qs = reinterpret_cast<T*>(smem + Lz::oQ);
  T* Wn = reinterpret_cast<T*>(smem + Lz::oW);
  T* Ks = reinterpret_cast<T*>(smem + Lz::oK);
  T* Os = reinterpret_cast<T*>(smem + Lz::oO);
  T* Tpp = reinterpret_cast<T*>(smem + Lz::oT);
  T* Pl = reinterpret_cast<T*>(smem + Lz::oP);
  const GateLds G = gate_lds(smem + Lz::oG);

  const FwdArgs& f = a.f;
  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  const int seg = seg0 + blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int b = bh / f.H, h = bh % f.H;
  const int blk0 = seg * f.L, blk1 = min(f.nblk, blk0 + f.L);
  const size_t rs = (size_t)f.H * D;
  const T* q = tok_base<T, D>(f.q, f.T, f.H, b, h);
  const T* k = tok_base<T, D>(f.k, f.T, f.H, b, h);
  const T* dO = tok_base<T, D>(a.dO, f.T, f.H, b, h);
  const float* al = f.alpha + (size_t)b * f.T * f.H + h;
  const float* bt = f.beta + (size_t)b * f.T * f.H + h;

  f32x4 dSv[DKT];
  {
    const float* G0 = (MAIN && dSend) ? dSend + ((size_t)bh * dsend_P + seg) * D * D : nullptr;
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa)
      dSv[aa] = G0 ? *reinterpret_cast<const f32x4*>(G0 + (size_t)(16 * w + li) * D + 16 * aa + g4)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  ScanPrefetch<T, D> pf;
  {
    const int t0 = (blk1 - 1) * BLK;
    pf.fetch(q, k, dO, al, bt, tp_block<T>(f.tw, f.nblk, bh, blk1 - 1), rs, f.H, t0,
             min(BLK, f.T - t0));
  }
  for (int blk = blk1 - 1; blk >= blk0; --blk) {
    const int t0 = blk * BLK, nv = min(BLK, f.T - t0);
    pf.stage(Qs, Ks, Os, Tpp, LDD, LDC, nv, G);
    if constexpr (MAIN)
      StateTiles<T, D>::store(reinterpret_cast<T*>(a.dhst) + ((size_t)bh * f.nblk + blk) * D * D,
                              w, lane, dSv);
    // the previous block's inputs, in three parts over the first half of this one
    const bool more = blk > blk0;
    auto fetch_part = [&](auto part) {
      pf.template fetch<decltype(part)::value>(q, k, dO, al, bt,
                                               tp_block<T>(f.tw, f.nblk, bh, blk - 1), rs, f.H,
                                               t0 - BLK, BLK);
    };
    if (more) fetch_part(std::integral_constant<int, 1>{});
    lds_barrier();
    // P scores, the dO^T diag(gamma) Q term and Wn = -Tpp diag(gamma) K
    block_scores<T, D, NW, true, false>(Qs, Ks, LDD, G, nullptr, 0, Pl, LDC);
    if (more) fetch_part(std::integral_constant<int, 2>{});
    f32x4 X2[DKT];
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) X2[aa] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto bo = frag_tr_gamma<T>(Os + 16 * w, LDD, s, G.gam);
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa)
        X2[aa] = Mma<T>::mma(frag_tr<T, STD>(Qs + 16 * aa, LDD, s), bo, X2[aa]);
    }
    if constexpr (Lz::W_IN_Q) lds_barrier();  // Q read before W replaces it
    block_w<T, D, NW>(Ks, LDD, Tpp, LDC, Wn, G.gam);
    lds_barrier();
    if (more) fetch_part(std::integral_constant<int, 4>{});
    // dVn = P^T dO + D (K dS'^T)
    f32x4 dvn[4], kd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dvn[i] = kd[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto bo = frag_tr<T, STD>(Os + 16 * w, LDD, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) dvn[i] = Mma<T>::mma(frag_tr<T, STD>(Pl + 16 * i, LDC, s), bo, dvn[i]);
    }
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
      const auto bs = AccFrag<T>::get(dSv, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) kd[i] = Mma<T>::mma(frag_row<T, PERM>(Ks + 16 * i * LDD, LDD, s), bs, kd[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dvn[i][e] += G.dec[16 * i + g4 + e] * kd[i][e];
    // dS = gamma_C dS' + dO^T diag(gamma) Q - dVn^T W   (Wn holds -W)
    const float gc = G.gC[0];
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) dSv[aa] = gc * dSv[aa] + X2[aa];
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto bv = AccFrag<T>::get(dvn, s);
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa)
        dSv[aa] = Mma<T>::mma(frag_tr<T, PERM>(Wn + 16 * aa, LDD, s), bv, dSv[aa]);
    }
    lds_barrier();
  }

  float* out = MAIN ? ((seg == 0 && a.dS_in) ? a.dS_in + (size_t)bh * D * D : nullptr)
                    : a.NBseg + ((size_t)bh * f.P + seg) * D * D;
  if (out) {
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa)
      *reinterpret_cast<f32x4*>(out + (size_t)(16 * w + li) * D + 16 * aa + g4) = dSv[aa];
  }
}

// The reverse scan with two blocks in flight (where its LDS plan fits, bf16):
// the state-free work of the next block in the walk (P, dO^T diag(gamma) Q
// and Wn) runs in the same barrier phase as the state work of the current
// one, on double-buffered K, dO, P, Wn and gates, so a block takes two
// barrier phases instead of three.  Each product is formed as in
// gdn_bwd_dscan_kernel, which remains for layouts that do not fit (fp32).
// Padded rows (no swizzle), as in the segment summary: 8-byte row pairs
// and transpose reads dominate here.
template <typename T, int D> struct Scan2Lds {
  static constexpr int LDD = D + Lay<T>::PADX;
  static constexpr int LDC = BLK + Lay<T>::PADX;
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t sq = (size_t)BLK * LDC * sizeof(T);
  static constexpr size_t oQ = 0, oT = oQ + rowD, oK = oT + sq, oO = oK + 2 * rowD,
                          oW = oO + 2 * rowD, oP = oW + 2 * rowD, oG = oP + 2 * sq;
  static constexpr size_t bytes = oG + 2 * kGateBytes;
  static constexpr bool fits = bytes <= 160 * 1024;
};

template <typename T, int D, bool MAIN>
__global__ __launch_bounds__(4 * D, 2) void gdn_bwd_dscan2_kernel(BwdArgs a, int seg0, int nseg,
                                                                  const float* dSend,
                                                                  int dsend_P) {
  typedef Scan2Lds<T, D> Lz;
  constexpr int DKT = D / 16, NW = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC;
  extern __shared__ __align__(16) unsigned char smem[];
  T* Qs = reinterpret_cast<T*>(smem + Lz::oQ);
  T* Tpp = reinterpret_cast<T*>(smem + Lz::oT);
  auto Kb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oK + n * Lz::rowD); };
  auto Ob = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oO + n * Lz::rowD); };
  auto Wb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oW + n * Lz::rowD); };
  auto Pb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oP + n * Lz::sq); };
  auto Gb = [&](int n) { return gate_lds(smem + Lz::oG + n * kGateBytes); };

  const FwdArgs& f = a.f;
  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  const int seg = seg0 + blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int b = bh / f.H, h = bh % f.H;
  const int blk0 = seg * f.L, blk1 = min(f.nblk, blk0 + f.L);
  const size_t rs = (size_t)f.H * D;
  const T* q = tok_base<T, D>(f.q, f.T, f.H, b, h);
  const T* k = tok_base<T, D>(f.k, f.T, f.H, b, h);
  const T* dO = tok_base<T, D>(a.dO, f.T, f.H, b, h);
  const float* al = f.alpha + (size_t)b * f.T * f.H + h;
  const float* bt = f.beta + (size_t)b * f.T * f.H + h;

  f32x4 dSv[DKT];
  {
    const float* G0 = (MAIN && dSend) ? dSend + ((size_t)bh * dsend_P + seg) * D * D : nullptr;
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa)
      dSv[aa] = G0 ? *reinterpret_cast<const f32x4*>(G0 + (size_t)(16 * w + li) * D + 16 * aa + g4)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  ScanPrefetch<T, D> pf;
  auto fetch = [&](int blk) {
    pf.fetch(q, k, dO, al, bt, tp_block<T>(f.tw, f.nblk, bh, blk), rs, f.H, blk * BLK,
             min(BLK, f.T - blk * BLK));
  };
  auto fetch_part = [&](auto part, int blk) {
    pf.template fetch<decltype(part)::value>(q, k, dO, al, bt, tp_block<T>(f.tw, f.nblk, bh, blk),
                                             rs, f.H, blk * BLK, BLK);
  };
  // State-free work of the block staged in Q, K[n], dO[n], Tpp and gates G[n]:
  // P -> P[n], X2 = dO^T diag(gamma) Q (registers), Wn = -Tpp diag(gamma) K -> W[n].
  f32x4 X2[DKT];
  auto pre = [&](int n) {
    const GateLds Gn = Gb(n);
    block_scores<T, D, NW, true, false>(Qs, Kb(n), LDD, Gn, nullptr, 0, Pb(n), LDC);
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) X2[aa] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto bo = frag_tr_gamma<T>(Ob(n) + 16 * w, LDD, s, Gn.gam);
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa)
        X2[aa] = Mma<T>::mma(frag_tr<T, STD>(Qs + 16 * aa, LDD, s), bo, X2[aa]);
    }
    block_w<T, D, NW>(Kb(n), LDD, Tpp, LDC, Wb(n), Gn.gam);
  };

  if (blk0 < blk1) {
    fetch(blk1 - 1);
    pf.stage(Qs, Kb(0), Ob(0), Tpp, LDD, LDC, min(BLK, f.T - (blk1 - 1) * BLK), Gb(0));
    if (blk1 - 2 >= blk0) fetch(blk1 - 2);
    lds_barrier();
    pre(0);
    lds_barrier();
  }
  for (int blk = blk1 - 1; blk >= blk0; --blk) {
    const int c = (blk1 - 1 - blk) & 1, n = c ^ 1;
    const bool next = blk > blk0, next2 = blk - 1 > blk0;
    if constexpr (MAIN)
      StateTiles<T, D>::store(reinterpret_cast<T*>(a.dhst) + ((size_t)bh * f.nblk + blk) * D * D,
                              w, lane, dSv);
    // This block's first operands (its buffers were published by the last
    // barrier), read before the next block's staging so that their LDS
    // latency overlaps it (bf16: dscan 154 -> 148 us, dscan summary 146 -> 140
    // us per launch on the benchmark).
    constexpr bool RA = sizeof(T) == 2;
    typename Mma<T>::frag rbo, rp[4], rk[4];
    if constexpr (RA) {
      rbo = frag_tr<T, STD>(Ob(c) + 16 * w, LDD, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rp[i] = frag_tr<T, STD>(Pb(c) + 16 * i, LDC, 0);
        rk[i] = frag_row<T, PERM>(Kb(c) + 16 * i * LDD, LDD, 0);
      }
    }
    // the next block (blk - 1) into the other buffers; the one after it goes
    // out in three parts over this block
    if (next) {
      pf.stage(Qs, Kb(n), Ob(n), Tpp, LDD, LDC, BLK, Gb(n));
      if (next2) fetch_part(std::integral_constant<int, 1>{}, blk - 2);
    }
    lds_barrier();
    // block blk: dVn = P^T dO + D (K dS'^T); dS = gamma_C dS' + X2 - dVn^T W
    {
      const GateLds Gc = Gb(c);
      f32x4 dvn[4], kd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dvn[i] = kd[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
        const auto bo = (RA && s == 0) ? rbo : frag_tr<T, STD>(Ob(c) + 16 * w, LDD, s);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dvn[i] = Mma<T>::mma((RA && s == 0) ? rp[i] : frag_tr<T, STD>(Pb(c) + 16 * i, LDC, s),
                               bo, dvn[i]);
      }
#pragma unroll
      for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
        const auto bs = AccFrag<T>::get(dSv, s);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          kd[i] = Mma<T>::mma((RA && s == 0) ? rk[i] : frag_row<T, PERM>(Kb(c) + 16 * i * LDD, LDD, s),
                              bs, kd[i]);
      }
      if (next2) fetch_part(std::integral_constant<int, 2>{}, blk - 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) dvn[i][e] += Gc.dec[16 * i + g4 + e] * kd[i][e];
      const float gc = Gc.gC[0];
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa) dSv[aa] = gc * dSv[aa] + X2[aa];
#pragma unroll
      for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
        const auto bv = AccFrag<T>::get(dvn, s);
#pragma unroll
        for (int aa = 0; aa < DKT; ++aa)
          dSv[aa] = Mma<T>::mma(frag_tr<T, PERM>(Wb(c) + 16 * aa, LDD, s), bv, dSv[aa]);
      }
    }
    // block blk - 1, state-free part
    if (next) pre(n);
    if (next2) fetch_part(std::integral_constant<int, 4>{}, blk - 2);
    lds_barrier();
  }

  float* out = MAIN ? ((seg == 0 && a.dS_in) ? a.dS_in + (size_t)bh * D * D : nullptr)
                    : a.NBseg + ((size_t)bh * f.P + seg) * D * D;
  if (out) {
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa)
      *reinterpret_cast<f32x4*>(out + (size_t)(16 * w + li) * D + 16 * aa + g4) = dSv[aa];
  }
}

static hipError_t set_lds(const void* fn, size_t bytes);

// The reverse scan over nseg segments from seg0, in the two-block form where it fits.
template <typename T, int D, bool MAIN>
static hipError_t launch_dscan(const BwdArgs& a, int seg0, int nseg, const float* dSend,
                               int dsend_P, hipStream_t st) {
  const int grid = a.f.B * a.f.H * nseg;
  constexpr size_t lds2 = Scan2Lds<T, D>::bytes, lds1 = ScanLds<T, D>::bytes;
  if constexpr (Scan2Lds<T, D>::fits) {
    hipError_t e = set_lds((const void*)gdn_bwd_dscan2_kernel<T, D, MAIN>, Scan2Lds<T, D>::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_bwd_dscan2_kernel<T, D, MAIN>), dim3(grid), dim3(4 * D),
                       lds2, st, a, seg0, nseg, dSend, dsend_P);
  } else {
    hipError_t e = set_lds((const void*)gdn_bwd_dscan_kernel<T, D, MAIN>, ScanLds<T, D>::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_bwd_dscan_kernel<T, D, MAIN>), dim3(grid), dim3(4 * D),
                       lds1, st, a, seg0, nseg, dSend, dsend_P);
  }
  return hipGetLastError();
}

// -------------------------------------------------------- block gradients ---
// Sums of a 16x16 accumulator tile C[m][n] (lane: m = 4 g + e, n = i):
// over n for each m (result valid in lanes with i == 0, element e), and over
// m for each n (result valid in lanes 0..15).
__device__ __forceinline__ f32x4 tile_sum_over_n(f32x4 v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = sum_row16(v[e]);
  return v;
}
__device__ __forceinline__ float tile_sum_over_m(f32x4 v) {
  return sum_rows4((v[0] + v[1]) + (v[2] + v[3]));
}

// fp32 operands of the gate-chain products (dT T^T and T^T Y, 64 x 64 x 64)
// go through the bf16 matrix cores as split tiles: x ~ hi + lo with
// hi = bf16(x) and lo = bf16(x - hi), about 16 significant bits.  A split
// tile row holds hi[64] | lo[64], SPLIT_LD bf16 = 256 bytes, swizzled like
// any 256-byte bf16 row.
constexpr int SPLIT_LD = 2 * BLK;
__device__ __forceinline__ void split_store(bf16* row, int c, float x) {
  const bf16 h = (bf16)x;
  *lds_sw(row + c, SPLIT_LD) = h;
  *lds_sw(row + BLK + c, SPLIT_LD) = (bf16)(x - (float)h);
}
// C += A B^T with both operands split, dropping only the lo*lo term.
__device__ __forceinline__ f32x4 mma_split(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
  c = Mma<bf16>::mma(al, bh, c);
  c = Mma<bf16>::mma(ah, bl, c);
  return Mma<bf16>::mma(ah, bh, c);
}
// *p += x in LDS without waiting for the old value (ds_add_f32).  The partial
// arrays are per wave, so the order of the additions is this wave's program
// order and the sums stay deterministic.
__device__ __forceinline__ void lds_add(float* p, float x) {
  __hip_atomic_fetch_add(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// part[m0 + m] += sum over n   (one writer lane per entry)
__device__ __forceinline__ void add_rows(float* part, int m0, f32x4 v, float sign = 1.f) {
  v = tile_sum_over_n(v);
  const int lane = lane_id();
  if ((lane & 15) == 0) {
    float* p = part + m0 + 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) lds_add(p + e, sign * v[e]);
  }
}
// part[n0 + n] += sum over m
__device__ __forceinline__ void add_cols(float* part, int n0, f32x4 v, float sign = 1.f) {
  const float x = tile_sum_over_m(v);
  const int lane = lane_id();
  if (lane < 16) lds_add(part + n0 + lane, sign * x);
}

// Pair terms of d log alpha.  A term X_rs (s <= r, one block) that carries the
// gate ratio Gamma_rs = exp(g_r - g_s) moves d log alpha_i for s < i <= r: the
// gradient of g_r minus that of g_s.  Summed as those two per-token sums and a
// suffix sum over the block, the terms with i <= s cancel only up to rounding,
// which leaves an error of the block's scale in d log alpha_i; where alpha_i is
// tiny, d log alpha_i = alpha_i dL/dalpha_i is tiny too and dalpha = d log
// alpha / alpha is lost.  Summed over the rectangle s < i <= r instead, every
// term of d log alpha_i contains alpha_i as a factor, so the sum keeps its
// relative accuracy.  pair_rect adds, for one 16 x 16 tile (row tile a =
// r-tile, column tile b = s-tile, b <= a) and every i, the tile's share of
// the rectangle sum to F[i] (this wave's partial, 64 floats): column
// prefixes for i inside the s-tile, the whole tile for i between the tiles,
// row suffixes for i inside the r-tile, and both for a diagonal tile.  Every
// partial sum adds only terms of its own rectangle.  Layout SR: lane (i, g)
// holds X[16a + i][16b + 4g + e]; RS: X[16a + 4g + e][16b + i].
// The gradient kernel sums a block's pair terms over rectangles where some
// alpha of the block is below this.  Above it the per-token sums were measured
// within 7e-6 (fp32) of the head's largest dalpha, and bf16 within its
// operands' own rounding (3e-3); below it they lose accuracy as 1/alpha.
constexpr float kRectAlpha = 0.02f;
template <bool SR>
__device__ __forceinline__ void pair_rect(float* F, int a, int b, const f32x4& v) {
  const int lane = lane_id(), li = lane & 15, g = lane >> 4;
  if (b > a) return;
  if (b < a) {
    float full;  // the tile's sum
    if constexpr (SR) {
      f32x4 cp;
#pragma unroll
      for (int e = 0; e < 4; ++e) cp[e] = sum_row16(v[e]);
      cp[1] += cp[0];
      cp[2] += cp[1];
      cp[3] += cp[2];
      const float t0 = lane_f(cp[3], 0), t1 = lane_f(cp[3], 16), t2 = lane_f(cp[3], 32),
                  t3 = lane_f(cp[3], 48);
      const float off = g == 0 ? 0.f : g == 1 ? t0 : g == 2 ? t0 + t1 : (t0 + t1) + t2;
      if (li == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lds_add(F + 16 * b + 4 * g + e + 1, off + cp[e]);
      }
      full = ((t0 + t1) + t2) + t3;
      // row suffixes: rows rho >= i of the whole tile
      float x = sum_rows4((v[0] + v[1]) + (v[2] + v[3]));
      x += dpp_f<0x101>(x);
      x += dpp_f<0x102>(x);
      x += dpp_f<0x104>(x);
      x += dpp_f<0x108>(x);
      if (g == 0 && li >= 1) lds_add(F + 16 * a + li, x);
    } else {
      float x = sum_rows4((v[0] + v[1]) + (v[2] + v[3]));  // column sum, sigma = li
      x += dpp_f<0x111>(x);
      x += dpp_f<0x112>(x);
      x += dpp_f<0x114>(x);
      x += dpp_f<0x118>(x);
      if (g == 0) lds_add(F + 16 * b + li + 1, x);
      full = lane_f(x, 15);
      f32x4 q;  // row sums, suffix over rho: in the lane over e, then the higher row groups
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = sum_row16(v[e]);
      q[2] += q[3];
      q[1] += q[2];
      q[0] += q[1];
      const float t1 = lane_f(q[0], 16), t2 = lane_f(q[0], 32), t3 = lane_f(q[0], 48);
      const float up = g == 3 ? 0.f : g == 2 ? t3 : g == 1 ? t2 + t3 : t1 + (t2 + t3);
      if (li == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g + e >= 1) lds_add(F + 16 * a + 4 * g + e, up + q[e]);
      }
    }
    // whole tile for 16 b + 16 < i <= 16 a
    if (lane < 16 * (a - b - 1)) lds_add(F + 16 * b + 17 + lane, full);
  } else {
    // diagonal tile: sum over rho >= k, sigma < k for k = 1 .. 15
    if constexpr (SR) {
      f32x4 p = v;  // row prefixes over this lane's 4 columns
      p[1] += p[0];
      p[2] += p[1];
      p[3] += p[2];
      const float u0 = __shfl(p[3], li), u1 = __shfl(p[3], li + 16), u2 = __shfl(p[3], li + 32);
      const float off = g == 0 ? 0.f : g == 1 ? u0 : g == 2 ? u0 + u1 : (u0 + u1) + u2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * g + e + 1;
        const float d = sum_row16(li >= k ? off + p[e] : 0.f);
        if (li == 0 && k <= 15) lds_add(F + 16 * a + k, d);
      }
    } else {
      f32x4 q = v;  // column suffixes over this lane's 4 rows
      q[2] += q[3];
      q[1] += q[2];
      q[0] += q[1];
      const float u1 = __shfl(q[0], li + 16), u2 = __shfl(q[0], li + 32), u3 = __shfl(q[0], li + 48);
      const float up = g == 3 ? 0.f : g == 2 ? u3 : g == 1 ? u2 + u3 : u1 + (u2 + u3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * g + e;
        const float d = sum_row16(li < k ? up + q[e] : 0.f);
        if (li == 0 && k >= 1) lds_add(F + 16 * a + k, d);
      }
    }
  }
}

// LDS plan of the gradient kernel (regions reused by phase):
//   RQ Q | RK K | RV V -> Y | RO dO -> dW | RT Tm | RA Af -> Tp, Tpp (-> dVn, dKK
//   for fp32 at d = 64) | RP P -> dPm | RW Vn -> dT | RD dVn -> dKK |
//   gates, per-wave partial sums.
// FAR (fp32 operands at d = 128, where the 64 x 128 tiles are 33 KiB each):
// RQ, RK, RV and RO lie in a global area of the workgroup instead of LDS,
// which holds the rest (142 KiB).
template <typename T, int D> struct GradLds {
  static constexpr int NW = D / 16;
  static constexpr int LDD = D + Lay<T>::PAD;
  static constexpr int LDC = BLK + Lay<T>::PADC;
  static constexpr int LDF = BLK + 4;
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t f64x64 = (size_t)BLK * LDF * sizeof(float);
  static constexpr size_t sq64 = (size_t)BLK * LDC * sizeof(T);
  // dVn fits the Tpp half of RA for fp32 at d = 64 only
  static constexpr bool DVN_IN_A = sizeof(T) == 4 && sq64 >= rowD;
  static constexpr bool BF = sizeof(T) == 2;  // swizzled bf16 tiles: regions 4 KiB aligned,
                                              // split tiles in place of the fp32 Y and dT
  static constexpr size_t al(size_t x) { return BF ? lds_align(x) : x; }
  static constexpr size_t zSplit = (size_t)BLK * 2 * BLK * 2;  // a split tile (64 rows x 256 B)
  static constexpr size_t zR = BF ? cmax(rowD, zSplit) : cmax(rowD, f64x64);
  static constexpr size_t zA = cmax(f64x64, 2 * sq64);
  static constexpr size_t zW = BF ? cmax(rowD, zSplit) : cmax(rowD, f64x64);
  static constexpr size_t zD = DVN_IN_A ? 0 : cmax(rowD, sq64);
  static constexpr size_t zPart = (4 * NW * BLK + NW + 4) * sizeof(float);
  // the input regions, from the start of their area (LDS, or the global area)
  static constexpr size_t oQ = 0, oK = oQ + zR, oV = oK + zR, oO = oV + zR, zIn = oO + zR;
  static constexpr size_t rest(size_t o0) {
    return al(al(al(al(o0 + f64x64) + zA) + sq64) + zW) + zD + kGateBytes + zPart;
  }
  static constexpr bool FAR = rest(zIn) > 160 * 1024;
  static constexpr size_t far_bytes = FAR ? zIn : 0;
  static constexpr size_t oT = FAR ? 0 : zIn, oA = al(oT + f64x64), oP = al(oA + zA),
                          oW = al(oP + sq64), oD = al(oW + zW), oG = oD + zD,
                          oPart = oG + kGateBytes;
  static constexpr size_t bytes = oPart + zPart;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(!BF || (oK % 4096 == 0 && oV % 4096 == 0 && oO % 4096 == 0 && oA % 4096 == 0 &&
                        oP % 4096 == 0 && oW % 4096 == 0 && oD % 4096 == 0),
                "swizzled tiles 4 KiB aligned");
  static_assert(!DVN_IN_A || sq64 >= rowD, "dVn must fit the Tpp half");
  // a [D][LDD] copy of the state fits V+dO and W+dVn (adjacent regions)
  static constexpr size_t zS = (size_t)D * LDD * sizeof(T);
  static_assert(zIn - oV >= zS && (oD + zD) - oW >= zS, "state copies");
};

// The gradients of block id (of B*H*nblk, the heads of one token block
// consecutive).  smem: the workgroup's LDS; in: the area of the input regions
// (smem, or the workgroup's global area when FAR).
template <typename T, int D>
__device__ __forceinline__ void grads_block(const BwdArgs& a, int id, unsigned char* smem,
                                            unsigned char* in) {
  typedef GradLds<T, D> Lz;
  constexpr int NW = Lz::NW, DKT = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC, LDF = Lz::LDF;
  constexpr int NJ = 16 / NW;  // 64x64 tiles per wave
  // With the input regions in global memory, a barrier must also publish
  // the global stores (the regions in LDS need only the LDS one).
  auto bar = [] {
    if constexpr (Lz::FAR) full_barrier();
    else lds_barrier();
  };
  T* Qs = reinterpret_cast<T*>(in + Lz::oQ);
  T* Ks = reinterpret_cast<T*>(in + Lz::oK);
  T* Vs = reinterpret_cast<T*>(in + Lz::oV);
  float* Yf = reinterpret_cast<float*>(in + Lz::oV);
  T* Os = reinterpret_cast<T*>(in + Lz::oO);
  T* dWs = reinterpret_cast<T*>(in + Lz::oO);
  float* Tm = reinterpret_cast<float*>(smem + Lz::oT);
  float* Af = reinterpret_cast<float*>(smem + Lz::oA);
  T* Tp = reinterpret_cast<T*>(smem + Lz::oA);
  T* Tpp = Tp + BLK * LDC;
  T* Pl = reinterpret_cast<T*>(smem + Lz::oP);
  T* Vns = reinterpret_cast<T*>(smem + Lz::oW);
  float* dTf = reinterpret_cast<float*>(smem + Lz::oW);
  T* dVns = Lz::DVN_IN_A ? Tpp : reinterpret_cast<T*>(smem + Lz::oD);
  T* dKKs = dVns;
  const GateLds G = gate_lds(smem + Lz::oG);
  float* part = reinterpret_cast<float*>(smem + Lz::oPart);

  const FwdArgs& f = a.f;
  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  float* dgp = part + w * BLK;                // dg per token, this wave's share
  float* dbp = part + NW * BLK + w * BLK;     // dbeta per token
  float* ddp = part + 2 * NW * BLK + w * BLK; // dD per token
  float* dfp = part + 3 * NW * BLK + w * BLK; // pair-term rectangle sums per token (pair_rect)
  float* dgc = part + 4 * NW * BLK;           // per-wave <dS', S>
  // Consecutive workgroups take the heads of one token block, so the rows
  // of [B, T, H, D] that run concurrently are read whole (H * D elements).
  const int BH = f.B * f.H;
  const int blk = id / BH, bh = id % BH;
  const int b = bh / f.H, h = bh % f.H;
  const int t0 = blk * BLK, nv = min(BLK, f.T - t0);
  const size_t rs = (size_t)f.H * D;
  const T* q = tok_base<T, D>(f.q, f.T, f.H, b, h) + (size_t)t0 * rs;
  const T* k = tok_base<T, D>(f.k, f.T, f.H, b, h) + (size_t)t0 * rs;
  const T* v = tok_base<T, D>(f.v, f.T, f.H, b, h) + (size_t)t0 * rs;
  const T* dO = tok_base<T, D>(a.dO, f.T, f.H, b, h) + (size_t)t0 * rs;
  T* dq = const_cast<T*>(tok_base<T, D>(a.dq, f.T, f.H, b, h)) + (size_t)t0 * rs;
  T* dk = const_cast<T*>(tok_base<T, D>(a.dk, f.T, f.H, b, h)) + (size_t)t0 * rs;
  T* dv = const_cast<T*>(tok_base<T, D>(a.dv, f.T, f.H, b, h)) + (size_t)t0 * rs;
  const size_t gofs = (size_t)b * f.T * f.H + (size_t)t0 * f.H + h;
  const T* hS = reinterpret_cast<const T*>(a.hst) + ((size_t)bh * f.nblk + blk) * D * D;
  const T* hG = reinterpret_cast<const T*>(a.dhst) + ((size_t)bh * f.nblk + blk) * D * D;
  // Vn of this block as the forward formed it (this wave's dv-tile)
  const T* hV = reinterpret_cast<const T*>(f.vst) + ((size_t)bh * f.nblk + blk) * BLK * D;

  // ---- A: Q, K and the gates, then the states (by dv-tile, first used in
  // phase C); V and dO (first used after the solve) go out at the start of
  // the solve and stay in flight in registers until then.  Each group of loads is
  // issued once the previous one's data is needed or staged, so that no wave
  // stalls issuing loads it will not use for a while ahead of those it needs
  // first (the address unit takes a workgroup's 128 KB at about 64 bytes per
  // cycle); issue order is wait order (vmcnt counts in order).
  typedef Tile<T, D, 4 * D> Tl;
  uint4 r2[Tl::NCH], r3[Tl::NCH];
  f32x4 Sx[DKT], dSx[DKT];  // by dv-tile: m = dk-tile, n = dv-tile w
  // alpha of this lane's token, kept for dalpha at the end (no global load
  // there: it would wait for every store of the block, vmcnt being in order)
  const float ra = f.alpha[gofs + (size_t)min(lane, nv - 1) * f.H];
  {
    const float rb = f.beta[gofs + (size_t)min(lane, nv - 1) * f.H];
    uint4 r0[Tl::NCH], r1[Tl::NCH];
    Tl::load(r0, q, rs, nv);
    Tl::load(r1, k, rs, nv);
    for (int i = threadIdx.x; i < 4 * NW * BLK + NW + 4; i += 64 * NW) part[i] = 0.f;
    Tl::to_lds(r0, Qs, LDD, nv);
    Tl::to_lds(r1, Ks, LDD, nv);
    if (w == 0) {
      block_gates(lane < nv ? __logf(ra) : 0.f, lane < nv ? rb : 0.f, G);
      const bool tiny = __ballot(lane < nv && ra < kRectAlpha) != 0;
      if (lane == 0) G.gC[2] = tiny ? 1.f : 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
    StateTiles<T, D>::load(hS, w, lane, Sx);
    StateTiles<T, D>::load(hG, w, lane, dSx);
    __builtin_amdgcn_sched_barrier(0);
  }
  bar();
  // the pair terms of d log alpha as rectangle sums (pair_rect) where the
  // block has a small alpha, else as per-token sums (the same value up to
  // rounding, and cheaper)
  const bool rect = __builtin_amdgcn_readfirstlane(G.gC[2] != 0.f ? 1 : 0) != 0;
  // ---- B: scores
  f32x4 kk[NJ];  // K K^T tiles (m = 16 (w & 3), n = 16 ((w >> 2) NJ + j)), for phase L
  block_scores<T, D, NW, true>(Qs, Ks, LDD, G, Af, LDF, Pl, LDC, kk);
  bar();
  // ---- C: T = (I + A)^{-1}, Tp, Tpp; zero Tm's upper blocks (solve scratch).
  // Meanwhile S and dS' go through LDS once, so that every wave also holds
  // them by dk-tile (S^T, dS'^T rows 16 w .. as operands over dv, for dQ, dW
  // and dK2): copies [dv][dk] in the V/dO and W/dVn regions, which are free
  // until V, dO are staged and W is formed.
  T* Sc = reinterpret_cast<T*>(in + Lz::oV);
  T* Gc = reinterpret_cast<T*>(smem + Lz::oW);
#pragma unroll
  for (int aa = 0; aa < DKT; ++aa) {
    const int off = (16 * w + li) * LDD + 16 * aa + g4;
    st4(lds_sw(Sc + off, LDD), Sx[aa][0], Sx[aa][1], Sx[aa][2], Sx[aa][3]);
    st4(lds_sw(Gc + off, LDD), dSx[aa][0], dSx[aa][1], dSx[aa][2], dSx[aa][3]);
  }
  if constexpr (Lz::FAR) vm_wait();  // the S copy is global: stored before the solve's barrier
  __builtin_amdgcn_sched_barrier(0);
  Tl::load(r2, v, rs, nv);
  Tl::load(r3, dO, rs, nv);
  uint4 rvn[StateTiles<T, BLK>::NV];
  StateTiles<T, BLK>::load_raw(hV, w, lane, rvn);
  __builtin_amdgcn_sched_barrier(0);
  // K dS'^T (this wave's dv-tile), for dVn in phase E: it needs only K and
  // dS', so it runs while the last wave does the substitution (and that wave
  // runs it during the first block step)
  f32x4 kd[4];
  auto kd_side = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) kd[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
      const auto bs = AccFrag<T>::get(dSx, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kd[i] = Mma<T>::mma(frag_row<T, PERM>(Ks + 16 * i * LDD, LDD, s), bs, kd[i]);
    }
  };
  block_solve<NW - 1>(Af, Tm, LDF, kd_side);  // its first barrier publishes the copies
  constexpr int KST = D / Mma<T>::KSTEP;
  typename Mma<T>::frag skf[KST], gkf[KST];
#pragma unroll
  for (int s = 0; s < KST; ++s) {
    skf[s] = frag_tr<T, STD>(Sc + 16 * w, LDD, s);
    gkf[s] = frag_tr<T, STD>(Gc + 16 * w, LDD, s);
  }
  block_tprime<T, 64 * NW, true>(Tm, LDF, G, Tp, Tpp, LDC);
  bar();  // copies read before V, dO and Vn replace them
  Tl::to_lds(r2, Vs, LDD, nv);
  Tl::to_lds(r3, Os, LDD, nv);
  {
    f32x4 vx[4];
    StateTiles<T, BLK>::unpack(rvn, vx);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_tile_N(vx[i], Vns, LDD, 16 * i, 16 * w);
  }
  bar();
  for (int i = threadIdx.x; i < BLK * BLK; i += 64 * NW) {
    const int r = i >> 6, s = i & 63;
    if ((s >> 4) > (r >> 4)) Tm[r * LDF + s] = 0.f;
  }
  // ---- E: <dS', S> of this wave's rows (for the gate of the block end)
  {
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) p += Sx[aa] * dSx[aa];
    const float x = wave_sum((p[0] + p[1]) + (p[2] + p[3]));
    if (lane == 0) dgc[w] = x;
  }
  // dVn = P^T dO + D (K dS'^T)
  f32x4 dvn[4];
  {
#pragma unroll
    for (int i = 0; i < 4; ++i) dvn[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto bo = frag_tr<T, STD>(Os + 16 * w, LDD, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) dvn[i] = Mma<T>::mma(frag_tr<T, STD>(Pl + 16 * i, LDC, s), bo, dvn[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dvn[i][e] += G.dec[16 * i + g4 + e] * kd[i][e];
  }
  // dV^T = dVn^T Tpp  (m = dv, n = s)
  {
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto av = AccFrag<T>::get(dvn, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = Mma<T>::mma(av, frag_tr<T, PERM>(Tpp + 16 * j, LDC, s), acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * j + li;
      if (r < nv) st4(dv + (size_t)r * rs + 16 * w + g4, acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    }
  }
  // ---- F: dVn to LDS.  Where dVn takes the Tpp tile (fp32 at d = 64) every
  // wave's reads of Tpp above come first; elsewhere its region is free, and
  // the barrier below alone keeps phase G's writes of dPm behind the reads of
  // P above.
  if constexpr (Lz::DVN_IN_A) bar();
#pragma unroll
  for (int i = 0; i < 4; ++i) store_tile_N(dvn[i], dVns, LDD, 16 * i, 16 * w);
  bar();
  // Operands read ahead (bf16, where registers are spare): phase H's dO
  // fragments here, phase I's first two k-steps of dVn and Vn fragments at the
  // start of H.  Their LDS reads then overlap the phase before instead of
  // stalling every wave at once after the barrier (gdn_bwd_grads 722 -> 710 us
  // per launch on the benchmark).
  constexpr bool READ_AHEAD = sizeof(T) == 2;
  typename Mma<T>::frag hO[READ_AHEAD ? D / Mma<T>::KSTEP : 1][4];
  if constexpr (READ_AHEAD) {
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) hO[s][j] = frag_row<T, STD>(Os + 16 * j * LDD, LDD, s);
  }
  // ---- G: dP^T (m = s, n = r) = Vn dO^T ; P-term of d log alpha ; dPm = dP o Gamma o mask in place of P
  {
    const int st = w & 3, r0 = (w >> 2) * NJ;
    f32x4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
      const auto av = frag_row<T, STD>(Vns + 16 * st * LDD, LDD, s);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[j] = Mma<T>::mma(av, frag_row<T, STD>(Os + 16 * (r0 + j) * LDD, LDD, s), acc[j]);
    }
    const int s0 = 16 * st + g4;
    f32x4 pg[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = 16 * (r0 + j) + li;
      T* pp = lds_sw(Pl + r * LDC + s0, LDC);  // 4 elements of one 16-byte chunk
      f32x4 dm;
      const float gr = G.g[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const float p = (float)pp[e];
        pg[j][e] = acc[j][e] * p;
        dm[e] = (s <= r) ? acc[j][e] * __expf(gr - G.g[s]) : 0.f;
      }
      st4(pp, dm[0], dm[1], dm[2], dm[3]);
    }
    if (rect) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) pair_rect<true>(dfp, r0 + j, st, pg[j]);
    } else {
      f32x4 pgs = {0.f, 0.f, 0.f, 0.f};  // pg summed over this wave's r-tiles
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        add_cols(dgp, 16 * (r0 + j), pg[j], 1.f);  // dg_r += sum_s
        pgs += pg[j];
      }
      add_rows(dgp, 16 * st, pgs, -1.f);  // dg_s -= sum_r
    }
  }
  bar();
  constexpr int NPI = READ_AHEAD ? 2 : 1;
  typename Mma<T>::frag iV[NPI][2][4];
  if constexpr (READ_AHEAD) {
#pragma unroll
    for (int s = 0; s < NPI; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        iV[s][0][j] = frag_row<T, STD>(dVns + 16 * j * LDD, LDD, s);
        iV[s][1][j] = frag_row<T, STD>(Vns + 16 * j * LDD, LDD, s);
      }
  }
  // ---- H: dQ^T = diag-scaled (S^T dO^T) + K^T dPm^T  (wave: dk-tile w); dK^T starts
  f32x4 dKt[4];
  {
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = dKt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (READ_AHEAD) acc[j] = Mma<T>::mma(skf[s], hO[s][j], acc[j]);
        else acc[j] = Mma<T>::mma(skf[s], frag_row<T, STD>(Os + 16 * j * LDD, LDD, s), acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * j + li;
      acc[j] *= G.gam[r];
      // O-term of dg: dg_r += sum_dk Q[r][dk] dQ1[r][dk]
      f32x4 qv;
      const T* qr = lds_sw(Qs + r * LDD + 16 * w + g4, LDD);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[e] = (float)qr[e] * acc[j][e];
      add_cols(dgp, 16 * j, qv, 1.f);
    }
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto ak = frag_tr<T, STD>(Ks + 16 * w, LDD, s);
      const auto aq = frag_tr<T, STD>(Qs + 16 * w, LDD, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto bp = frag_tr<T, STD>(Pl + 16 * j, LDC, s);   // dPm^T rows
        acc[j] = Mma<T>::mma(ak, frag_row<T, STD>(Pl + 16 * j * LDC, LDC, s), acc[j]);
        dKt[j] = Mma<T>::mma(aq, bp, dKt[j]);                    // dK1 = Q^T dPm
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * j + li;
      if (r < nv) st4(dq + (size_t)r * rs + 16 * w + g4, acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    }
  }
  // dW takes the dO region.  Where dO's operands were read ahead (bf16), every
  // read of dO ended before phase G's barrier; else phase H reads dO from LDS,
  // and this barrier keeps dW out until every wave has.
  if constexpr (!READ_AHEAD) bar();
  // ---- I: dW^T = -(S^T dVn^T) -> dW row-major ; dK2^T = dS'^T Vn^T scaled by D ; D-term
  {
    f32x4 acc[4], x2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = x2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (READ_AHEAD && s < NPI) {
          acc[j] = Mma<T>::mma(skf[s], iV[s < NPI ? s : 0][0][j], acc[j]);
          x2[j] = Mma<T>::mma(gkf[s], iV[s < NPI ? s : 0][1][j], x2[j]);
        } else {
          acc[j] = Mma<T>::mma(skf[s], frag_row<T, STD>(dVns + 16 * j * LDD, LDD, s), acc[j]);
          x2[j] = Mma<T>::mma(gkf[s], frag_row<T, STD>(Vns + 16 * j * LDD, LDD, s), x2[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      store_tile_T(acc[j], dWs, LDD, 16 * w, 16 * j, -1.f);
      const int s = 16 * j + li;
      f32x4 kv;
      const T* kr = lds_sw(Ks + s * LDD + 16 * w + g4, LDD);
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[e] = (float)kr[e] * x2[j][e];
      add_cols(ddp, 16 * j, kv, 1.f);
      dKt[j] += G.dec[s] * x2[j];
    }
  }
  bar();
  // ---- J: dTp = dW K^T, dTpp = dVn V^T (m = r, n = s); dT; column terms
  // (bf16: T also goes to a split tile in the Q region, free after phase H)
  constexpr bool SPLIT = sizeof(T) == 2;
  bf16* Tx = reinterpret_cast<bf16*>(in + Lz::oQ);    // T, split
  bf16* dTx = reinterpret_cast<bf16*>(smem + Lz::oW);  // dT, split (in place of dTf)
  bf16* YTx = reinterpret_cast<bf16*>(in + Lz::oV);   // Y^T, split (in place of Yf)
  static_assert(Lz::zR >= BLK * SPLIT_LD * 2 && Lz::zW >= BLK * SPLIT_LD * 2, "split tiles");
  if constexpr (SPLIT) {
    // eight consecutive elements per thread: one 16-byte chunk of hi and one
    // of lo (the swizzle moves whole chunks)
    for (int i = threadIdx.x; i < BLK * BLK / 8; i += 64 * NW) {
      const int r = i >> 3, c0 = 8 * (i & 7);
      bf16x8 h, l;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = Tm[r * LDF + c0 + e];
        h[e] = (bf16)x;
        l[e] = (bf16)(x - (float)h[e]);
      }
      *reinterpret_cast<bf16x8*>(lds_sw(Tx + r * SPLIT_LD + c0, SPLIT_LD)) = h;
      *reinterpret_cast<bf16x8*>(lds_sw(Tx + r * SPLIT_LD + BLK + c0, SPLIT_LD)) = l;
    }
  }
  {
    const int rt = w & 3, s0t = (w >> 2) * NJ;
    f32x4 a1[NJ], a2[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) a1[j] = a2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / Mma<T>::KSTEP; ++s) {
      const auto aw = frag_row<T, STD>(dWs + 16 * rt * LDD, LDD, s);
      const auto au = frag_row<T, STD>(dVns + 16 * rt * LDD, LDD, s);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        a1[j] = Mma<T>::mma(aw, frag_row<T, STD>(Ks + 16 * (s0t + j) * LDD, LDD, s), a1[j]);
        a2[j] = Mma<T>::mma(au, frag_row<T, STD>(Vs + 16 * (s0t + j) * LDD, LDD, s), a2[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int s = 16 * (s0t + j) + li;
      const float bg = G.bg[s], bs = G.beta[s], gs = G.gam[s];
      f32x4 dt, c1, c2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + g4 + e;
        const bool low = s <= r;
        const float tv = low ? Tm[r * LDF + s] : 0.f;
        dt[e] = low ? a1[j][e] * bg + a2[j][e] * bs : 0.f;
        c1[e] = a1[j][e] * tv;  // d(beta gamma)_s
        c2[e] = a2[j][e] * tv;  // dbeta_s through Tpp
      }
      if constexpr (SPLIT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) split_store(dTx + (16 * rt + g4 + e) * SPLIT_LD, s, dt[e]);
      } else {
        store_tile_N(dt, dTf, LDF, 16 * rt, 16 * (s0t + j));
      }
      const float sbg = tile_sum_over_m(c1), sb2 = tile_sum_over_m(c2);
      if (lane < 16) {
        lds_add(dbp + s, sb2 + gs * sbg);
        lds_add(dgp + s, bs * gs * sbg);
      }
    }
  }
  bar();
  // ---- K: Y = dT T^T (fp32 products; split tiles for bf16)
  {
    const int rt = w & 3, s0t = (w >> 2) * NJ;
    f32x4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (SPLIT) {
      const bf16* pa = dTx + 16 * rt * SPLIT_LD;
#pragma unroll
      for (int s = 0; s < BLK / Mma<bf16>::KSTEP; ++s) {
        const bf16x8 ah = frag_row<bf16, STD>(pa, SPLIT_LD, s);
        const bf16x8 al = frag_row<bf16, STD>(pa + BLK, SPLIT_LD, s);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16* pb = Tx + 16 * (s0t + j) * SPLIT_LD;
          acc[j] = mma_split(ah, al, frag_row<bf16, STD>(pb, SPLIT_LD, s),
                             frag_row<bf16, STD>(pb + BLK, SPLIT_LD, s), acc[j]);
        }
      }
      // Y^T[s'][r .. r+3], split
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        bf16* row = YTx + (16 * (s0t + j) + li) * SPLIT_LD + 16 * rt + g4;
        bf16x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = (bf16)acc[j][e];
          l[e] = (bf16)(acc[j][e] - (float)h[e]);
        }
        *reinterpret_cast<bf16x4*>(lds_sw(row, SPLIT_LD)) = h;
        *reinterpret_cast<bf16x4*>(lds_sw(row + BLK, SPLIT_LD)) = l;
      }
    } else {
#pragma unroll
      for (int s = 0; s < BLK / 4; ++s) {
        const float av = frag_row<float, STD>(dTf + 16 * rt * LDF, LDF, s);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[j] = Mma<float>::mma(av, frag_row<float, STD>(Tm + 16 * (s0t + j) * LDF, LDF, s), acc[j]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) store_tile_N(acc[j], Yf, LDF, 16 * rt, 16 * (s0t + j));
    }
  }
  bar();
  // ---- L: dA = -T^T Y (strictly lower); A-terms of dbeta and d log alpha; dKK + dKK^T
  {
    const int rt = w & 3, s0t = (w >> 2) * NJ;
    f32x4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (SPLIT) {
#pragma unroll
      for (int s = 0; s < BLK / Mma<bf16>::KSTEP; ++s) {
        const bf16x8 ah = frag_tr<bf16, STD>(Tx + 16 * rt, SPLIT_LD, s);
        const bf16x8 al = frag_tr<bf16, STD>(Tx + BLK + 16 * rt, SPLIT_LD, s);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16* pb = YTx + 16 * (s0t + j) * SPLIT_LD;
          acc[j] = mma_split(ah, al, frag_row<bf16, STD>(pb, SPLIT_LD, s),
                             frag_row<bf16, STD>(pb + BLK, SPLIT_LD, s), acc[j]);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < BLK / 4; ++s) {
        const float at = frag_tr<float, STD>(Tm + 16 * rt, LDF, s);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[j] = Mma<float>::mma(at, frag_tr<float, STD>(Yf + 16 * (s0t + j), LDF, s), acc[j]);
      }
    }
    // db's row sums, over this wave's s-tiles, give the dbeta_r term and
    // (times beta_r) the row term of dg, or the pair terms beta_r db_rs go to
    // the rectangle sums
    f32x4 dbr = {0.f, 0.f, 0.f, 0.f}, dag[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int s = 16 * (s0t + j) + li;
      const float gs = G.g[s];
      f32x4 db, dkk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + g4 + e;
        const bool low = s < r;
        const float gam = low ? __expf(G.g[r] - gs) : 0.f;
        const float da = low ? -acc[j][e] : 0.f;
        const float br = G.beta[r];
        db[e] = da * gam * kk[j][e];
        dag[j][e] = br * db[e];
        dkk[e] = da * br * gam;
      }
      // dKK + dKK^T in place of dKK (dKK is strictly lower, so the two never
      // overlap): a tile on or below the diagonal goes to its mirror
      // transposed, then its lower part to its place (on the diagonal, over
      // the zeros its transpose carried there); the tiles above the
      // diagonal are other waves' mirrors
      if (s0t + j <= rt) {
        store_tile_T(dkk, dKKs, LDC, 16 * rt, 16 * (s0t + j));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + g4 + e;
          if (s < r) *lds_sw(dKKs + r * LDC + s, LDC) = from_f<T>(dkk[e]);
        }
      }
      dbr += db;
    }
    if (rect) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) pair_rect<false>(dfp, rt, s0t + j, dag[j]);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) add_cols(dgp, 16 * (s0t + j), dag[j], -1.f);
    }
    dbr = tile_sum_over_n(dbr);
    if (li == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + g4 + e;
        lds_add(dbp + r, dbr[e]);
        if (!rect) lds_add(dgp + r, G.beta[r] * dbr[e]);
      }
    }
  }
  bar();
  // ---- N: gate gradients.  d log alpha_j collects the terms through gamma_r
  // for r >= j (dg: the O-term of dQ and the gamma of Tp), the terms through
  // D_i = exp(g_C - g_i) for i < j (dj), the state's decay gamma_C, and the
  // pair terms.  With the pair terms as rectangle sums each of these carries
  // alpha_j as a factor, so d log alpha_j keeps its relative accuracy however
  // small alpha_j is, and so does dalpha_j = d log alpha_j / alpha_j.  Else
  // (no alpha below kRectAlpha in the block) the pair terms are in dg, and
  // d log alpha is the suffix sum of dg with dj moved to the block's end.
  // Every term is in place after phase L, and phase M writes no LDS, so
  // wave 0 forms them ahead of its share of M, beside the other waves'
  // (the workgroup ends when its last wave does).
  if (w == 0) {
    // wave 0 ends last (the gates, then its share of dK): it goes ahead of
    // the wave it shares a SIMD with until the block's end
    __builtin_amdgcn_s_setprio(2);
    const int j = lane;
    float dg = 0.f, dbv = 0.f, dd = 0.f, gcs = 0.f, fr = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      dg += part[ww * BLK + j];
      dbv += part[NW * BLK + ww * BLK + j];
      dd += part[2 * NW * BLK + ww * BLK + j];
      fr += part[3 * NW * BLK + ww * BLK + j];
      gcs += dgc[ww];
    }
    const float dj = G.dec[j] * dd;
    float x;
    if (rect) {
      // dj of token j - 1 (the shuffle runs in every lane: a lane that sat
      // out would hand its neighbour nothing)
      const float dj_up = __shfl_up(dj, 1);
      const float dj_prev = j == 0 ? 0.f : dj_up;
      x = ((wave_suffix_sum(dg) + wave_prefix_sum(dj_prev)) + G.gC[0] * gcs) + fr;
    } else {
      dg -= dj;
      const float dgC = wave_sum(dj) + G.gC[0] * gcs;
      if (j == BLK - 1) dg += dgC;
      x = wave_suffix_sum(dg);  // dlog alpha_j = sum_{r >= j} dg_r
    }
    if (j < nv) {
      const size_t idx = gofs + (size_t)j * f.H;
      a.dalpha[idx] = x / ra;
      a.dbeta[idx] = dbv;
    }
  }
  // ---- M: dK^T += K^T (dKK + dKK^T) + dW^T Tp ; store dk
  {
#pragma unroll
    for (int s = 0; s < BLK / Mma<T>::KSTEP; ++s) {
      const auto ak = frag_tr<T, STD>(Ks + 16 * w, LDD, s);
      const auto aw = frag_tr<T, STD>(dWs + 16 * w, LDD, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dKt[j] = Mma<T>::mma(ak, frag_row<T, STD>(dKKs + 16 * j * LDC, LDC, s), dKt[j]);
        dKt[j] = Mma<T>::mma(aw, frag_tr<T, STD>(Tp + 16 * j, LDC, s), dKt[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 16 * j + li;
      if (s < nv) st4(dk + (size_t)s * rs + 16 * w + g4, dKt[j][0], dKt[j][1], dKt[j][2], dKt[j][3]);
    }
  }
  if (w == 0) __builtin_amdgcn_s_setprio(0);  // (the strided form runs further blocks)
}

template <typename T, int D>
__global__ __launch_bounds__(4 * D, 2) void gdn_bwd_grads_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  if constexpr (GradLds<T, D>::FAR) {
    // a grid of at most kFarGroups workgroups, each with its own global area,
    // striding over the blocks
    unsigned char* in = reinterpret_cast<unsigned char*>(a.far) + (size_t)blockIdx.x * GradLds<T, D>::far_bytes;
    const int n = a.f.B * a.f.H * a.f.nblk;
    for (int id = blockIdx.x; id < n; id += gridDim.x) {
      grads_block<T, D>(a, id, smem, in);
      full_barrier();  // every read of this block done before the next one's stores
    }
  } else {
    grads_block<T, D>(a, blockIdx.x, smem, smem);
  }
}

// ------------------------------------------------------------ launch -------
static hipError_t set_lds(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int D>
hipError_t launch_bwd(const BwdArgs& a0, bool saved, int phase, hipStream_t st, Profiler* prof) {
  BwdArgs a = a0;
  FwdArgs& f = a.f;
  const int BH = f.B * f.H, P = f.P;
  constexpr size_t grad_bytes = GradLds<T, D>::bytes;
  hipError_t e;
  if (phase != PHASE_ALL && !saved) return hipErrorInvalidValue;
  const bool begin = phase != PHASE_END, end = phase != PHASE_BEGIN;
  // 0. per-block Tp, Tpp (Pre)
  if (!saved && (e = launch_prep<T, D>(f, st, prof)) != hipSuccess) return e;
  const float* dSend = a.dS_out;
  int dsend_P = 1;
  if (P > 1) {
    // 1. segment maps of the forward (all segments)
    if (!saved && (e = launch_fwd_summary<T, D>(f, P, st, prof, "gdn_bwd_summary")) != hipSuccess)
      return e;
    // 2. NB maps of segments 1..P-1 (independent of dS_out)
    if (begin) {
      prof_begin(prof, "gdn_bwd_dscan_summary", st);
      e = launch_dscan<T, D, false>(a, 1, P - 1, nullptr, 1, st);
      prof_end(prof, st);
      if (e != hipSuccess) return e;
    }
    if (!end) return hipGetLastError();
    // 3. chains
    if (!saved) {
      ChainArgs c{f.S_in, f.Mseg, f.Nseg, const_cast<float*>(f.Sst), P, BH};
      if ((e = launch_chain<D, false>(c, st, prof)) != hipSuccess) return e;
    }
    ChainArgs cb{a.dS_out, f.MBseg, a.NBseg, a.dSend, P, BH};
    if ((e = launch_chain<D, true>(cb, st, prof)) != hipSuccess) return e;
    dSend = a.dSend;
    dsend_P = P;
  } else {
    if (!end) return hipSuccess;
    f.Sst = f.S_in;
    f.sst_P = 1;
  }
  // 4. block entry states and Vn
  if (!saved && (e = launch_states<T, D>(f, a.hst, st, prof)) != hipSuccess) return e;
  // 5. block exit gradients and dS_in
  prof_begin(prof, "gdn_bwd_dscan", st);
  e = launch_dscan<T, D, true>(a, 0, P, dSend, dsend_P, st);
  prof_end(prof, st);
  if (e != hipSuccess) return e;
  // 6. per-block gradients
  if ((e = set_lds((const void*)gdn_bwd_grads_kernel<T, D>, GradLds<T, D>::bytes)) != hipSuccess)
    return e;
  if (GradLds<T, D>::FAR && !a.far) return hipErrorInvalidValue;
  const int nblocks = BH * f.nblk;
  const int grid = GradLds<T, D>::FAR ? std::min(nblocks, kFarGroups) : nblocks;
  prof_begin(prof, "gdn_bwd_grads", st);
  hipLaunchKernelGGL((gdn_bwd_grads_kernel<T, D>), dim3(grid), dim3(4 * D), grad_bytes, st, a);
  prof_end(prof, st);
  return hipGetLastError();
}

size_t bwd_far_bytes(bool f32, int D) {
  if (!f32) return 0;
  return (D == 128 ? GradLds<float, 128>::far_bytes : GradLds<float, 64>::far_bytes) * kFarGroups;
}

template hipError_t launch_bwd<bf16, 128>(const BwdArgs&, bool, int, hipStream_t, Profiler*);
template hipError_t launch_bwd<bf16, 64>(const BwdArgs&, bool, int, hipStream_t, Profiler*);
template hipError_t launch_bwd<float, 128>(const BwdArgs&, bool, int, hipStream_t, Profiler*);
template hipError_t launch_bwd<float, 64>(const BwdArgs&, bool, int, hipStream_t, Profiler*);

}  // namespace sfgdn
