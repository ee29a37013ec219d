// Forward kernels of one pipeline chunk of the gated delta rule.
//
// A chunk of T tokens is nblk = ceil(T/64) kernel blocks per (batch, head).
// The blocks are grouped into P segments of L blocks.  Each block maps the
// state affinely, S' = S M_b + N_b with M_b = gamma_C I - W^T D K and
// N_b = U^T D K, so a segment is an affine map too.  The forward runs
//   0. gdn_prep:        per block, fully parallel, the state-free part of
//      Pre: T = (I + A)^{-1} and its scaled copy Tpp = T diag(beta) (the
//      only serial step inside a block, so it is kept out of the scan
//      kernels; Tp = Tpp diag(gamma) is applied through K where W is formed);
//   1. gdn_fwd_summary: per segment (except the last), its map (M, N) from
//      the identity and a zero state, fully parallel;
//   2. gdn_chain_fwd:   segment entry states S_{j+1} = S_j M_j + N_j, a short
//      serial chain that starts from S_in;
//   3. gdn_fwd_out:     per segment, from its true entry state, the fused
//      W/U, ST and Out pass over its blocks: outputs o, and S_out from the
//      last segment.
// This is the page's boundary-state chain (Eq. 5, Pith review of StateFlow,
// "What carries the argument") applied inside one chunk so that the low
// parallelism of the state transition (Figure 2 caption; "grid-size tuning")
// does not leave the GPU idle: P segments give B*H*P workgroups.
#include "gdn_kernels.hpp"

namespace sfgdn {

// ------------------------------------------------------------------ LDS ----
// One-block scan kernels (the forms used where the two-block plans below do
// not fit): one workgroup = D/16 waves, one per 16-column slice of the state.
// Regions:
//   RK : K (row-major; K^T operands come from transpose reads)
//   RV : V (row-major; V^T operands come from transpose reads)
//   RW : Wn = -W (for Vn)
//   RT : Tpp (from the Pre kernel)
//   RG : gate vectors
// and, for the out kernel only,
//   RQ : Q (P scores, S Q^T)
//   RP : P (masked decayed scores, for the output)
// The summary stops after RG.  Where the out kernel's plan would not fit
// otherwise (fp32 operands at d = 128: 64 x 128 fp32 tiles are 33 KiB), W
// shares V's region and RQ takes RW: U = Tpp V is then formed before W, with
// a barrier between.
template <typename T, int D> struct FwdLds {
  static constexpr int LDD = D + Lay<T>::PAD;
  static constexpr int LDC = BLK + Lay<T>::PADC;
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t sq = (size_t)BLK * LDC * sizeof(T);
  static constexpr size_t al(size_t x) { return sizeof(T) == 2 ? lds_align(x) : x; }
  static constexpr size_t oK = 0, oV = oK + rowD, oW = oV + rowD, oT = oW + rowD, oG = oT + sq;
  static constexpr size_t sum_bytes = oG + kGateBytes;
  static constexpr bool W_IN_V = al(sum_bytes) + rowD + sq > 160 * 1024;
  static constexpr size_t oWo = W_IN_V ? oV : oW;
  static constexpr size_t oQ = W_IN_V ? oW : al(sum_bytes);
  static constexpr size_t oP = W_IN_V ? al(sum_bytes) : oQ + rowD;
  static constexpr size_t out_bytes = oP + sq;
  static_assert(sum_bytes <= 160 * 1024 && out_bytes <= 160 * 1024, "LDS budget");
  static_assert(sizeof(T) != 2 || (oV % 4096 == 0 && oW % 4096 == 0 && oT % 4096 == 0 &&
                                   oQ % 4096 == 0 && oP % 4096 == 0), "swizzled tiles 4 KiB aligned");
};

// Fused out kernel, two blocks in flight: block b's state work (O += Vn^T P^T
// and the state update) reads K, P and gates of buffer b % 2 while block b+1
// forms P, S Q^T and Vn from the other buffer.  Q, V and Tpp are single: they
// are consumed in the iteration that stages them.
template <typename T, int D> struct OutLds {
  static constexpr int LDD = D + Lay<T>::PAD;
  static constexpr int LDC = BLK + Lay<T>::PAD;
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t sq = (size_t)BLK * LDC * sizeof(T);
  static constexpr size_t oQ = 0, oV = oQ + rowD, oT = oV + rowD, oK = oT + sq,
                          oP = oK + 2 * rowD, oG = oP + 2 * sq;
  static constexpr size_t bytes = oG + 2 * kGateBytes;
  static constexpr bool fits = bytes <= 160 * 1024;
  static_assert(sizeof(T) != 2 || (oV % 4096 == 0 && oT % 4096 == 0 && oK % 4096 == 0 &&
                                   oP % 4096 == 0), "swizzled tiles 4 KiB aligned");
};

// Pre kernel: one region holds K, then A (fp32; formed after every wave's K
// reads), then T, which the solve writes over A in place | RG gates.  About
// 19 KB at d = 128 in bf16, so eight workgroups share a CU (four with K and A
// in separate regions: 116 -> 92 us on the 65,536-token forward).
template <typename T, int D> struct PrepLds {
  static constexpr int LDD = D + Lay<T>::PAD;
  static constexpr int LDF = BLK + 4;
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t f64x64 = (size_t)BLK * LDF * sizeof(float);
  static constexpr size_t oK = 0, oT = 0, oA = 0, oG = cmax(rowD, f64x64);
  static constexpr size_t bytes = oG + kGateBytes;
};

// Token rows of one (b, h) sequence: row t starts at base + t * H * D.
template <typename T, int D>
__device__ __forceinline__ const T* seq_base(const void* p, const FwdArgs& a, int b, int h) {
  return reinterpret_cast<const T*>(p) + ((size_t)b * a.T * a.H + h) * D;
}


// Per-block inputs in flight: the next block's rows (q, k, v), its Tpp
// from the Pre kernel and its gates are loaded into registers while the
// current block computes.
// Vn of block blk of sequence bh in a.vst: 64 x D values in tile order.
template <typename T, int D>
__device__ __forceinline__ T* vn_block(const FwdArgs& a, int bh, int blk) {
  return reinterpret_cast<T*>(a.vst) + ((size_t)bh * a.nblk + blk) * BLK * D;
}

// Waves per workgroup of the forward kernels: one per 16-column tile of the
// state.
template <int D> constexpr int fwd_nw() { return D / 16; }

// Tpp = T diag(beta) of block blk of sequence bh: [64][64] row-major (Tp =
// Tpp diag(gamma) is applied through K when W is formed).
template <typename T>
__device__ __forceinline__ const T* tw_block(const void* tw, int nblk, int bh, int blk) {
  return reinterpret_cast<const T*>(tw) + ((size_t)bh * nblk + blk) * BLK * BLK;
}

template <typename T, int D, bool WITH_Q> struct Prefetch {
  typedef Tile<T, D, 64 * fwd_nw<D>()> Tl;
  typedef Tile<T, BLK, 64 * fwd_nw<D>()> Tt;
  uint4 rq[WITH_Q ? Tl::NCH : 1], rk[Tl::NCH], rv[Tl::NCH], rpp[Tt::NCH];
  float ra = 1.f, rb = 0.f;  // raw gates of the next block (wave 0)
  // PART: 1 the gates and Tpp, 2 q and k, 4 v (bit mask).  Spreading the
  // parts over a block keeps the address unit's time for them beside the
  // matrix work instead of stalling every wave at once.
  template <int PART = 7>
  __device__ __forceinline__ void fetch(const T* q, const T* k, const T* v, const float* al,
                                        const float* bt, const T* tw, size_t rs, int H, int t0,
                                        int nv) {
    if constexpr (PART & 1) {
      if (wave_id() == 0) {
        const size_t idx = (size_t)(t0 + min(lane_id(), nv - 1)) * H;
        ra = al[idx];
        rb = bt[idx];
      }
      Tt::load(rpp, tw, BLK, BLK);
    }
    if constexpr (PART & 2) {
      if constexpr (WITH_Q) Tl::load(rq, q + (size_t)t0 * rs, rs, nv);
      Tl::load(rk, k + (size_t)t0 * rs, rs, nv);
    }
    if constexpr (PART & 4) Tl::load(rv, v + (size_t)t0 * rs, rs, nv);
  }
  __device__ __forceinline__ void stage(T* Qs, T* Ks, T* Vs, T* Tpp, int ld, int ldc, int nv,
                                        const GateLds& G) {
    Tt::to_lds(rpp, Tpp, ldc, BLK);
    if constexpr (WITH_Q) Tl::to_lds(rq, Qs, ld, nv);
    Tl::to_lds(rk, Ks, ld, nv);
    Tl::to_lds(rv, Vs, ld, nv);
    if (wave_id() == 0) {
      const bool ok = lane_id() < nv;
      block_gates(ok ? __logf(ra) : 0.f, ok ? rb : 0.f, G);
    }
  }
};

// ------------------------------------------------------------ Pre ----------
// One workgroup of 4 waves per 64-token block, every block of every sequence
// in parallel: gates, A = strict lower part of diag(beta) (K K^T o Gamma),
// T = (I + A)^{-1} (fp32), then Tpp = T diag(beta) in the operand type to
// tw[b*H + h][block][64][64] (the kernels that form W = Tp K apply
// Tp = Tpp diag(gamma) through K).
template <typename T, int D>
__global__ __launch_bounds__(256) void gdn_prep_kernel(FwdArgs a) {
  typedef PrepLds<T, D> Lz;
  constexpr int LDD = Lz::LDD, LDF = Lz::LDF;
  extern __shared__ __align__(16) unsigned char smem[];
  T* Ks = reinterpret_cast<T*>(smem + Lz::oK);
  float* Af = reinterpret_cast<float*>(smem + Lz::oA);
  float* Tm = reinterpret_cast<float*>(smem + Lz::oT);
  const GateLds G = gate_lds(smem + Lz::oG);

  // consecutive workgroups: the heads of one token block (whole rows of k)
  const int BH = a.B * a.H;
  const int blk = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int b = bh / a.H, h = bh % a.H;
  const int t0 = blk * BLK, nv = min(BLK, a.T - t0);
  const size_t rs = (size_t)a.H * D;
  typedef Tile<T, D, 256> Tl;
  uint4 rk[Tl::NCH];
  Tl::load(rk, seq_base<T, D>(a.k, a, b, h) + (size_t)t0 * rs, rs, nv);
  float ra = 1.f, rb = 0.f;
  if (wave_id() == 0) {
    const size_t idx = (size_t)b * a.T * a.H + (size_t)(t0 + min(lane_id(), nv - 1)) * a.H + h;
    ra = a.alpha[idx];
    rb = a.beta[idx];
  }
  Tl::to_lds(rk, Ks, LDD, nv);
  if (wave_id() == 0) {
    const bool ok = lane_id() < nv;
    block_gates(ok ? __logf(ra) : 0.f, ok ? rb : 0.f, G);
  }
  lds_barrier();
  block_scores<T, D, 4, false, true, true>(nullptr, Ks, LDD, G, Af, LDF, nullptr, 0);
  lds_barrier();
  block_solve(Af, Tm, LDF);
  T* out = const_cast<T*>(tw_block<T>(a.tw, a.nblk, bh, blk));
  block_tprime<T, 256, false>(Tm, LDF, G, nullptr, out, BLK);
}

// --------------------------------------------------------- fused out -------
// Wave w owns dv-tiles NDV*w .. of the state: S^T, U/Vn and O^T for those
// columns live in its registers for the whole segment.  MODE selects what is
// written: OUT_ONLY the outputs o (and S_out); STATES_ONLY each block's entry
// state ([dv][dk], rounded to the operand type T, which is the precision the
// state has wherever it enters a product) to hst[b*H + h][block] and no
// output; OUT_AND_STATES both.  The backward consumes the stored states.
enum FwdMode { OUT_ONLY = 0, STATES_ONLY = 1, OUT_AND_STATES = 2 };

template <typename T, int D, int MODE>
__global__ __launch_bounds__(64 * fwd_nw<D>(), 2) void gdn_fwd_out_kernel(FwdArgs a, T* hst) {
  typedef FwdLds<T, D> Lz;
  constexpr int NW = fwd_nw<D>(), NDV = D / 16 / NW, DKT = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC;
  constexpr bool STATES = MODE != OUT_ONLY, OUT = MODE != STATES_ONLY;
  constexpr bool PFQ = sizeof(T) == 2;  // operand prefetch: registers allow it for bf16
  extern __shared__ __align__(16) unsigned char smem[];
  T* Qs = reinterpret_cast<T*>(smem + Lz::oQ);
  T* Ks = reinterpret_cast<T*>(smem + Lz::oK);
  T* Vs = reinterpret_cast<T*>(smem + Lz::oV);
  T* Wn = reinterpret_cast<T*>(smem + Lz::oWo);
  T* Tpp = reinterpret_cast<T*>(smem + Lz::oT);
  T* Pl = reinterpret_cast<T*>(smem + Lz::oP);
  const GateLds G = gate_lds(smem + Lz::oG);

  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  const int dv0 = NDV * w;
  const int seg = blockIdx.x % a.P, bh = blockIdx.x / a.P;
  const int b = bh / a.H, h = bh % a.H;
  const int blk0 = seg * a.L, blk1 = min(a.nblk, blk0 + a.L);
  const size_t rs = (size_t)a.H * D;
  const T* q = seq_base<T, D>(a.q, a, b, h);
  const T* k = seq_base<T, D>(a.k, a, b, h);
  const T* v = seq_base<T, D>(a.v, a, b, h);
  T* o = const_cast<T*>(seq_base<T, D>(a.o, a, b, h));
  const float* al = a.alpha + (size_t)b * a.T * a.H + h;
  const float* bt = a.beta + (size_t)b * a.T * a.H + h;

  // State S^T tiles: St[bb][aa] covers dk-tile aa, dv-tile dv0 + bb.
  f32x4 St[NDV][DKT];
  {
    const float* S0 = a.Sst ? a.Sst + ((size_t)bh * a.sst_P + seg) * D * D : nullptr;
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa) {
        const int dv = 16 * (dv0 + bb) + li, dk = 16 * aa + g4;
        St[bb][aa] = S0 ? *reinterpret_cast<const f32x4*>(S0 + (size_t)dv * D + dk)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }

  Prefetch<T, D, OUT> pf;
  if (blk0 < blk1)
    pf.fetch(q, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk0), rs, a.H, blk0 * BLK,
             min(BLK, a.T - blk0 * BLK));
  f32x4 O[NDV][4];
  int prev_t0 = -1, prev_nv = 0;
  auto store_o = [&]() {
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * j + li;
        if (r < prev_nv) {
          const f32x4 x = O[bb][j];
          st4(o + (size_t)(prev_t0 + r) * rs + 16 * (dv0 + bb) + g4, x[0], x[1], x[2], x[3]);
        }
      }
  };

  for (int blk = blk0; blk < blk1; ++blk) {
    const int t0 = blk * BLK, nv = min(BLK, a.T - t0);
    pf.stage(Qs, Ks, Vs, Tpp, LDD, LDC, nv, G);
    if constexpr (STATES) {
      static_assert(NDV == 1, "one state tile row per wave");
      StateTiles<T, D>::store(hst + ((size_t)bh * a.nblk + blk) * D * D, dv0, lane, St[0]);
    }
    if constexpr (OUT) {
      if (prev_t0 >= 0) store_o();
    }
    lds_barrier();
    // P = masked Q K^T o Gamma; O^T = diag(gamma) S Q^T; Wn = -Tpp diag(gamma) K; U = Tpp V
    if constexpr (OUT) {
      block_scores<T, D, NW, true, false>(Qs, Ks, LDD, G, nullptr, 0, Pl, LDC);
      zero_acc(O);
      block_s_yT<T, D, NDV>(St, Qs, LDD, O);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gr = G.gam[16 * j + li];
#pragma unroll
        for (int bb = 0; bb < NDV; ++bb) O[bb][j] *= gr;
      }
    }
    f32x4 U[NDV][4];
    block_u<T, NDV>(Tpp, LDC, Vs, LDD, dv0, U);
    if constexpr (Lz::W_IN_V) lds_barrier();  // V read before W replaces it
    block_w<T, D, NW>(Ks, LDD, Tpp, LDC, Wn, G.gam);
    lds_barrier();
    // ST and Out: Vn = U - W S^T; O^T += Vn^T P^T; S' = gamma_C S + Vn^T D K
    block_x_st<T, D, NDV, PFQ>(Wn, LDD, St, U);
    if constexpr (STATES)
      StateTiles<T, BLK>::store(vn_block<T, D>(a, bh, blk), dv0, lane, U[0]);
    if constexpr (OUT) block_vnT_pT<T, NDV, PFQ>(U, Pl, LDC, O);
    f32x4 dsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dsc[i][e] = G.dec[16 * i + g4 + e];
    const float gc = G.gC[0];
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa) St[bb][aa] *= gc;
    block_state_write<T, D, NDV, PFQ>(Ks, LDD, U, dsc, St);
    prev_t0 = t0;
    prev_nv = nv;
    // The next block's inputs: issued here so that they add no register
    // pressure to the phases above.
    if (blk + 1 < blk1)
      pf.fetch(q, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk + 1), rs, a.H, t0 + BLK,
               min(BLK, a.T - t0 - BLK));
    lds_barrier();
  }
  if constexpr (OUT) {
    if (prev_t0 >= 0) store_o();
  }

  if (OUT && seg == a.P - 1 && a.S_out) {
    float* So = a.S_out + (size_t)bh * D * D;
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa)
        *reinterpret_cast<f32x4*>(So + (size_t)(16 * (dv0 + bb) + li) * D + 16 * aa + g4) =
            St[bb][aa];
  }
}

// The same computation with two blocks in flight (OutLds): used where its
// LDS layout fits (bf16).
template <typename T, int D, int MODE>
__global__ __launch_bounds__(64 * fwd_nw<D>(), 2) void gdn_fwd_out2_kernel(FwdArgs a, T* hst) {
  typedef OutLds<T, D> Lz;
  constexpr int NW = fwd_nw<D>(), NDV = D / 16 / NW, DKT = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC;
  constexpr bool STATES = MODE != OUT_ONLY, OUT = MODE != STATES_ONLY;
  extern __shared__ __align__(16) unsigned char smem[];
  T* Qs = reinterpret_cast<T*>(smem + Lz::oQ);
  T* Vs = reinterpret_cast<T*>(smem + Lz::oV);
  T* Tpp = reinterpret_cast<T*>(smem + Lz::oT);
  // double buffers, by parity n
  auto Kb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oK + n * Lz::rowD); };
  auto Pb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oP + n * Lz::sq); };
  auto Gb = [&](int n) { return gate_lds(smem + Lz::oG + n * kGateBytes); };

  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  const int dv0 = NDV * w;
  const int seg = blockIdx.x % a.P, bh = blockIdx.x / a.P;
  const int b = bh / a.H, h = bh % a.H;
  const int blk0 = seg * a.L, blk1 = min(a.nblk, blk0 + a.L);
  const size_t rs = (size_t)a.H * D;
  const T* q = seq_base<T, D>(a.q, a, b, h);
  const T* k = seq_base<T, D>(a.k, a, b, h);
  const T* v = seq_base<T, D>(a.v, a, b, h);
  T* o = const_cast<T*>(seq_base<T, D>(a.o, a, b, h));
  const float* al = a.alpha + (size_t)b * a.T * a.H + h;
  const float* bt = a.beta + (size_t)b * a.T * a.H + h;

  // State S^T tiles: St[bb][aa] covers dk-tile aa, dv-tile dv0 + bb.
  f32x4 St[NDV][DKT];
  {
    const float* S0 = a.Sst ? a.Sst + ((size_t)bh * a.sst_P + seg) * D * D : nullptr;
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa) {
        const int dv = 16 * (dv0 + bb) + li, dk = 16 * aa + g4;
        St[bb][aa] = S0 ? *reinterpret_cast<const f32x4*>(S0 + (size_t)dv * D + dk)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }
  if (blk0 >= blk1) return;

  auto fetch = [&](Prefetch<T, D, OUT>& pf, int blk) {
    pf.fetch(q, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk), rs, a.H, blk * BLK,
             min(BLK, a.T - blk * BLK));
  };
  auto fetch_part = [&](auto part, Prefetch<T, D, OUT>& pf, int blk) {
    pf.template fetch<decltype(part)::value>(q, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk),
                                             rs, a.H, blk * BLK, min(BLK, a.T - blk * BLK));
  };
  // The state-free work of a block whose inputs sit in Q, K[n], V, Tpp and
  // gates G[n]: its masked decayed scores P -> P[n].
  auto block_p = [&](int n) {
    if constexpr (OUT) block_scores<T, D, NW, true, false>(Qs, Kb(n), LDD, Gb(n), nullptr, 0, Pb(n), LDC);
  };
  // With S the entry state of the block staged in Q, K[n], V, Tpp, G[n]:
  // O^T = diag(gamma) S Q^T and, from Z = K S^T in the same pass over the
  // state's fragments, Vn = U - W S^T = Tpp (V - diag(gamma) Z) -> U, since
  // W = Tpp diag(gamma) K.  No W tile is formed.
  f32x4 O[NDV][4];
  auto state_in_part = [&](int n, f32x4 (&U)[NDV][4]) {
    f32x4 Z[NDV][4];
    zero_acc(Z);
    zero_acc(O);
    block_s_kq<T, D, NDV, OUT>(St, Kb(n), Qs, LDD, Z, O);
    if constexpr (OUT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gr = Gb(n).gam[16 * j + li];
#pragma unroll
        for (int bb = 0; bb < NDV; ++bb) O[bb][j] *= gr;
      }
    }
    block_vn_from_z<T, NDV>(Tpp, LDC, Vs, LDD, dv0, Gb(n).gam, Z, U);
  };

  Prefetch<T, D, OUT> pf;
  fetch(pf, blk0);
  pf.stage(Qs, Kb(0), Vs, Tpp, LDD, LDC, min(BLK, a.T - blk0 * BLK), Gb(0));
  if (blk0 + 1 < blk1) fetch(pf, blk0 + 1);
  lds_barrier();
  f32x4 U[NDV][4];
  block_p(0);
  state_in_part(0, U);
  lds_barrier();

  for (int blk = blk0; blk < blk1; ++blk) {
    const int c = (blk - blk0) & 1, n = c ^ 1;
    const int t0 = blk * BLK, nv = min(BLK, a.T - t0);
    const bool next = blk + 1 < blk1;
    if constexpr (STATES) {
      static_assert(NDV == 1, "one state tile row per wave");
      StateTiles<T, D>::store(hst + ((size_t)bh * a.nblk + blk) * D * D, dv0, lane, St[0]);
    }
    const bool next2 = blk + 2 < blk1;
    if (next) {
      pf.stage(Qs, Kb(n), Vs, Tpp, LDD, LDC, min(BLK, a.T - t0 - BLK), Gb(n));
      if (next2) fetch_part(std::integral_constant<int, 1>{}, pf, blk + 2);
    }
    lds_barrier();
    // block blk, state part (U holds its Vn): O^T += Vn^T P^T; S' = gamma_C S + Vn^T D K
    if constexpr (STATES)
      StateTiles<T, BLK>::store(vn_block<T, D>(a, bh, blk), dv0, lane, U[0]);
    if (next2) fetch_part(std::integral_constant<int, 2>{}, pf, blk + 2);
    if constexpr (OUT) block_vnT_pT<T, NDV, true>(U, Pb(c), LDC, O);
    {
      f32x4 dsc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) dsc[i][e] = Gb(c).dec[16 * i + g4 + e];
      const float gc = Gb(c).gC[0];
#pragma unroll
      for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
        for (int aa = 0; aa < DKT; ++aa) St[bb][aa] *= gc;
      block_state_write<T, D, NDV, true>(Kb(c), LDD, U, dsc, St);
    }
    if (next2) fetch_part(std::integral_constant<int, 4>{}, pf, blk + 2);
    if constexpr (OUT) {
#pragma unroll
      for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * j + li;
          if (r < nv) {
            const f32x4 x = O[bb][j];
            st4(o + (size_t)(t0 + r) * rs + 16 * (dv0 + bb) + g4, x[0], x[1], x[2], x[3]);
          }
        }
    }
    // block blk+1: P, then S Q^T and Vn (S is now its entry state)
    if (next) {
      block_p(n);
      state_in_part(n, U);
    }
    lds_barrier();
  }

  if (OUT && seg == a.P - 1 && a.S_out) {
    float* So = a.S_out + (size_t)bh * D * D;
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa)
        *reinterpret_cast<f32x4*>(So + (size_t)(16 * (dv0 + bb) + li) * D + 16 * aa + g4) =
            St[bb][aa];
  }
}

// ------------------------------------------------------ segment summary ----
// Per segment: N = the exit state from a zero entry state and M = the product
// of the block maps M_b = gamma_C I - W^T D K, both fp32, row-major [D][D].
// Wave w owns rows NDV*w .. of N (dv) and of M (i); the propagation
//   M' = gamma_C M - (M W^T) D K
// runs like the state update with M in place of S.
template <typename T, int D>
__global__ __launch_bounds__(64 * fwd_nw<D>(), 2) void gdn_fwd_summary_kernel(FwdArgs a, int nseg) {
  typedef FwdLds<T, D> Lz;
  constexpr int NW = fwd_nw<D>(), NDV = D / 16 / NW, DKT = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC;
  extern __shared__ __align__(16) unsigned char smem[];
  T* Wn = reinterpret_cast<T*>(smem + Lz::oW);
  T* Ks = reinterpret_cast<T*>(smem + Lz::oK);
  T* Vs = reinterpret_cast<T*>(smem + Lz::oV);
  T* Tpp = reinterpret_cast<T*>(smem + Lz::oT);
  const GateLds G = gate_lds(smem + Lz::oG);

  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  const int dv0 = NDV * w;
  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int b = bh / a.H, h = bh % a.H;
  const int blk0 = seg * a.L, blk1 = min(a.nblk, blk0 + a.L);
  const size_t rs = (size_t)a.H * D;
  const T* k = seq_base<T, D>(a.k, a, b, h);
  const T* v = seq_base<T, D>(a.v, a, b, h);
  const float* al = a.alpha + (size_t)b * a.T * a.H + h;
  const float* bt = a.beta + (size_t)b * a.T * a.H + h;

  // NM[bb] holds N^T, NM[NDV + bb] holds M^T (tiles m = dk, n = dv): the two
  // maps go through every product together as 2 NDV state tiles, so each W
  // and K operand read from LDS serves both.
  f32x4 NM[2 * NDV][DKT];
#pragma unroll
  for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) {
      NM[bb][aa] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        NM[NDV + bb][aa][e] = (16 * aa + g4 + e == 16 * (dv0 + bb) + li) ? 1.f : 0.f;
    }

  Prefetch<T, D, false> pf;
  if (blk0 < blk1)
    pf.fetch(nullptr, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk0), rs, a.H, blk0 * BLK,
             min(BLK, a.T - blk0 * BLK));
  for (int blk = blk0; blk < blk1; ++blk) {
    const int t0 = blk * BLK, nv = min(BLK, a.T - t0);
    pf.stage(nullptr, Ks, Vs, Tpp, LDD, LDC, nv, G);
    lds_barrier();
    block_w<T, D, NW>(Ks, LDD, Tpp, LDC, Wn, G.gam);
    f32x4 X[NDV][4];
    block_u<T, NDV>(Tpp, LDC, Vs, LDD, dv0, X);
    lds_barrier();
    f32x4 dsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dsc[i][e] = G.dec[16 * i + g4 + e];
    const float gc = G.gC[0];
    // N: Vn0 = U - W N^T ; N' = gamma_C N + Vn0^T D K
    // M: Z = -(W M^T)    ; M' = gamma_C M + Z^T D K
    constexpr bool EARLY = sizeof(T) == 2;
    f32x4 X2[2 * NDV][4];
#pragma unroll
    for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        X2[bb][i] = X[bb][i];
        X2[NDV + bb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    block_x_st<T, D, 2 * NDV>(Wn, LDD, NM, X2);
#pragma unroll
    for (int bb = 0; bb < 2 * NDV; ++bb)
#pragma unroll
      for (int aa = 0; aa < DKT; ++aa) NM[bb][aa] *= gc;
    // The next block's inputs go out here, so that their latency is covered
    // by the state writes (for fp32 operands registers do not allow it).
    if (EARLY && blk + 1 < blk1)
      pf.fetch(nullptr, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk + 1), rs, a.H, t0 + BLK,
               min(BLK, a.T - t0 - BLK));
    block_state_write<T, D, 2 * NDV>(Ks, LDD, X2, dsc, NM);
    if (!EARLY && blk + 1 < blk1)
      pf.fetch(nullptr, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk + 1), rs, a.H, t0 + BLK,
               min(BLK, a.T - t0 - BLK));
    lds_barrier();
  }

  // NM holds N^T (m = dk, n = dv) -> N[dv][dk..] and M^T (m = j, n = i) -> M[i][j..].
  // The forward chain takes M transposed, the backward chain M row-major.
  float* MTo = a.Mseg + ((size_t)bh * a.P + seg) * D * D;
  float* No = a.Nseg + ((size_t)bh * a.P + seg) * D * D;
  float* Mo = a.MBseg ? a.MBseg + ((size_t)bh * a.P + seg) * D * D : nullptr;
#pragma unroll
  for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) {
      const size_t off = (size_t)(16 * (dv0 + bb) + li) * D + 16 * aa + g4;
      *reinterpret_cast<f32x4*>(No + off) = NM[bb][aa];
      if (Mo) *reinterpret_cast<f32x4*>(Mo + off) = NM[NDV + bb][aa];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        MTo[(size_t)(16 * aa + g4 + e) * D + 16 * (dv0 + bb) + li] = NM[NDV + bb][aa][e];
    }
}

// The segment summary with two blocks in flight (where its LDS plan fits,
// bf16): the next block's W and U are formed in the same barrier phase as
// the current block's map updates, on double-buffered K, W and gates, so a
// block takes two barrier phases instead of three.
// Padded rows (no swizzle): this kernel reads its W tile through 8-byte row
// pairs, which the padded layout lets the compiler fetch in one instruction.
template <typename T, int D> struct Sum2Lds {
  static constexpr int LDD = D + Lay<T>::PADX;
  static constexpr int LDC = BLK + Lay<T>::PADXC;
  static constexpr size_t rowD = (size_t)BLK * LDD * sizeof(T);
  static constexpr size_t sq = (size_t)BLK * LDC * sizeof(T);
  static constexpr size_t oV = 0, oT = oV + rowD, oK = oT + sq, oW = oK + 2 * rowD,
                          oG = oW + 2 * rowD;
  static constexpr size_t bytes = oG + 2 * kGateBytes;
  static constexpr bool fits = bytes <= 160 * 1024 && sizeof(T) == 2;
};

template <typename T, int D>
__global__ __launch_bounds__(64 * fwd_nw<D>(), 2) void gdn_fwd_summary2_kernel(FwdArgs a, int nseg) {
  typedef Sum2Lds<T, D> Lz;
  constexpr int NW = fwd_nw<D>(), NDV = D / 16 / NW, DKT = D / 16;
  constexpr int LDD = Lz::LDD, LDC = Lz::LDC;
  extern __shared__ __align__(16) unsigned char smem[];
  T* Vs = reinterpret_cast<T*>(smem + Lz::oV);
  T* Tpp = reinterpret_cast<T*>(smem + Lz::oT);
  auto Kb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oK + n * Lz::rowD); };
  auto Wb = [&](int n) { return reinterpret_cast<T*>(smem + Lz::oW + n * Lz::rowD); };
  auto Gb = [&](int n) { return gate_lds(smem + Lz::oG + n * kGateBytes); };

  const int w = wave_id(), lane = lane_id(), g4 = 4 * (lane >> 4), li = lane & 15;
  const int dv0 = NDV * w;
  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int b = bh / a.H, h = bh % a.H;
  const int blk0 = seg * a.L, blk1 = min(a.nblk, blk0 + a.L);
  const size_t rs = (size_t)a.H * D;
  const T* k = seq_base<T, D>(a.k, a, b, h);
  const T* v = seq_base<T, D>(a.v, a, b, h);
  const float* al = a.alpha + (size_t)b * a.T * a.H + h;
  const float* bt = a.beta + (size_t)b * a.T * a.H + h;

  // NM[bb] holds N^T, NM[NDV + bb] holds M^T (tiles m = dk, n = dv), as in
  // gdn_fwd_summary_kernel.
  f32x4 NM[2 * NDV][DKT];
#pragma unroll
  for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) {
      NM[bb][aa] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        NM[NDV + bb][aa][e] = (16 * aa + g4 + e == 16 * (dv0 + bb) + li) ? 1.f : 0.f;
    }

  Prefetch<T, D, false> pf;
  auto fetch = [&](int blk) {
    pf.fetch(nullptr, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk), rs, a.H, blk * BLK,
             min(BLK, a.T - blk * BLK));
  };
  auto fetch_part = [&](auto part, int blk) {
    pf.template fetch<decltype(part)::value>(nullptr, k, v, al, bt, tw_block<T>(a.tw, a.nblk, bh, blk),
                                             rs, a.H, blk * BLK, min(BLK, a.T - blk * BLK));
  };
  // state-free work of the block staged in K[n], V, Tpp and gates G[n]
  f32x4 U[NDV][4];
  auto pre = [&](int n) {
    block_w<T, D, NW>(Kb(n), LDD, Tpp, LDC, Wb(n), Gb(n).gam);
    block_u<T, NDV>(Tpp, LDC, Vs, LDD, dv0, U);
  };

  if (blk0 < blk1) {
    fetch(blk0);
    pf.stage(nullptr, Kb(0), Vs, Tpp, LDD, LDC, min(BLK, a.T - blk0 * BLK), Gb(0));
    if (blk0 + 1 < blk1) fetch(blk0 + 1);
    lds_barrier();
    pre(0);
    lds_barrier();
  }
  for (int blk = blk0; blk < blk1; ++blk) {
    const int c = (blk - blk0) & 1, n = c ^ 1;
    const bool next = blk + 1 < blk1, next2 = blk + 2 < blk1;
    // this block's first W operands (published by the last barrier), read
    // before the next block's staging so that their LDS latency overlaps it
    typename Mma<T>::frag rW[1][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rW[0][i] = frag_row<T, PERM>(Wb(c) + 16 * i * LDD, LDD, 0);
    if (next) {
      pf.stage(nullptr, Kb(n), Vs, Tpp, LDD, LDC, min(BLK, a.T - (blk + 1) * BLK), Gb(n));
      if (next2) fetch_part(std::integral_constant<int, 1>{}, blk + 2);
    }
    lds_barrier();
    // block blk:  N: Vn0 = U - W N^T ; N' = gamma_C N + Vn0^T D K
    //             M: Z = -(W M^T)    ; M' = gamma_C M + Z^T D K
    {
      const GateLds Gc = Gb(c);
      f32x4 dsc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) dsc[i][e] = Gc.dec[16 * i + g4 + e];
      const float gc = Gc.gC[0];
      f32x4 X2[2 * NDV][4];
#pragma unroll
      for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          X2[bb][i] = U[bb][i];
          X2[NDV + bb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      block_x_st_ra<T, D, 2 * NDV, 1>(Wb(c), LDD, NM, rW, X2);
#pragma unroll
      for (int bb = 0; bb < 2 * NDV; ++bb)
#pragma unroll
        for (int aa = 0; aa < DKT; ++aa) NM[bb][aa] *= gc;
      if (next2) fetch_part(std::integral_constant<int, 2>{}, blk + 2);
      block_state_write<T, D, 2 * NDV>(Kb(c), LDD, X2, dsc, NM);
    }
    // block blk + 1, state-free part
    if (next) pre(n);
    if (next2) fetch_part(std::integral_constant<int, 4>{}, blk + 2);
    lds_barrier();
  }

  float* MTo = a.Mseg + ((size_t)bh * a.P + seg) * D * D;
  float* No = a.Nseg + ((size_t)bh * a.P + seg) * D * D;
  float* Mo = a.MBseg ? a.MBseg + ((size_t)bh * a.P + seg) * D * D : nullptr;
#pragma unroll
  for (int bb = 0; bb < NDV; ++bb)
#pragma unroll
    for (int aa = 0; aa < DKT; ++aa) {
      const size_t off = (size_t)(16 * (dv0 + bb) + li) * D + 16 * aa + g4;
      *reinterpret_cast<f32x4*>(No + off) = NM[bb][aa];
      if (Mo) *reinterpret_cast<f32x4*>(Mo + off) = NM[NDV + bb][aa];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        MTo[(size_t)(16 * aa + g4 + e) * D + 16 * (dv0 + bb) + li] = NM[NDV + bb][aa][e];
    }
}

// ------------------------------------------------------------ chain ---------
// The boundary-state chain between segments, X' = X B_j + C_j for one
// sequence (Eq. 5 inside the chunk; its backward mirror, Eq. 7, for REV):
//   forward:  X_0 = S_in (or 0),   X_{j+1} = X_j M_j + N_j,      j = 0 .. P-2
//   backward: X_{P-1} = dS_out (or 0), X_{j-1} = X_j M_j^T + NB_j, j = P-1 .. 1
// All X are written to out[P][D][D].  Bt[j] holds B_j^T row-major (the
// transposed maps forward, the row-major maps backward) so that a lane's
// 8 contraction elements are contiguous.
//
// One workgroup per (sequence, 16 rows of X), D/16 waves, wave w owning
// output columns 16 w ..; the workgroups of one sequence on one XCD.  Each
// product runs on bf16 MFMA with the operands split into bf16 pairs, x = hi +
// lo, and the three terms hi*hi + hi*lo + lo*hi accumulated in fp32: about
// 2^-16 relative error per term, against fp32 MFMA at a quarter of the rate.
// The maps of the next two steps are in flight in registers while a step
// runs, so a step costs its MFMA chain and one LDS hand-off of X.
__device__ __forceinline__ void split_bf16(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 ha = (bf16)a[e], hb = (bf16)b[e];
    hi[e] = ha;
    hi[4 + e] = hb;
    lo[e] = (bf16)(a[e] - (float)ha);
    lo[4 + e] = (bf16)(b[e] - (float)hb);
  }
}

template <int D> struct ChainIn {
  static constexpr int KS = D / 32;
  f32x4 b[KS][2];  // B^T row (16 w + i), contraction 32 s + 8 g .. + 7
  float c[4];      // C rows r0 + 4 g + e, column 16 w + i
};

template <int D, bool REV>
__global__ __launch_bounds__(64 * (D / 16)) void gdn_chain_kernel(ChainArgs c) {
  constexpr int RT = D / 16, KS = D / 32, LDX = D + 8;
  __shared__ __align__(16) bf16 Xs[2][2][16 * LDX];  // [ping-pong][hi, lo] rows of X
  const int w = wave_id(), lane = lane_id(), g = lane >> 4;
  int bh, rt;
  xcd_seq_tile(blockIdx.x, RT, bh, rt);
  if (bh >= c.BH) return;
  const int P = c.P, r0 = 16 * rt, col = 16 * w + (lane & 15);
  const size_t DD = (size_t)D * D;
  const float* Bt = c.Bt + (size_t)bh * P * DD;
  const float* Cm = c.C + (size_t)bh * P * DD;
  float* out = c.out + (size_t)bh * P * DD;
  // this lane's 4 entries of the wave's 16x16 tile: rows r0 + 4 g + e, column col
  auto put = [&](int buf, int idx, const f32x4& x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * g + e;
      out[(size_t)idx * DD + (size_t)(r0 + m) * D + col] = x[e];
      const bf16 h = (bf16)x[e];
      Xs[buf][0][m * LDX + col] = h;
      Xs[buf][1][m * LDX + col] = (bf16)(x[e] - (float)h);
    }
  };
  const int nst = P - 1;
  // The map fetches are arranged so that a step waits only for its own
  // fetch (vmcnt counts in order):
  //  - a fetch is never conditional (a step past the end is clamped to the
  //    last one and unused), so the three ring buffers stay in place instead
  //    of being copied, which would wait for the loads in flight;
  //  - scheduling barriers keep each fetch's loads together, in order;
  //  - buffer loads with fixed per-lane byte offsets and a scalar step
  //    offset need no fresh vector address registers (reusing those would
  //    wait for the loads that last wrote them).  Offsets past the resource
  //    read zero instead of faulting.
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Bt), 0, (int)(P * DD * sizeof(float)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Cm), 0, (int)(P * DD * sizeof(float)), 0x00020000);
  const int boff = 4 * (col * D + 8 * g), coff = 4 * ((r0 + 4 * g) * D + col);
  auto fetch = [&](int i, ChainIn<D>& in) {
    __builtin_amdgcn_sched_barrier(0);
    i = min(i, nst - 1);
    const int so = (REV ? P - 1 - i : i) * (int)(DD * sizeof(float));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      in.b[s][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, boff + 128 * s, so, 0));
      in.b[s][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, boff + 128 * s + 16, so, 0));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      in.c[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rC, coff + 4 * D * e, so, 0));
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int i, const ChainIn<D>& in) {
    const bf16* Xh = Xs[i & 1][0];
    const bf16* Xl = Xs[i & 1][1];
    f32x4 a0 = {in.c[0], in.c[1], in.c[2], in.c[3]}, a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 xh = frag_row<bf16, STD>(Xh, LDX, s), xl = frag_row<bf16, STD>(Xl, LDX, s);
      bf16x8 bh8, bl8;
      split_bf16(in.b[s][0], in.b[s][1], bh8, bl8);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bh8, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bl8, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bh8, a2, 0, 0, 0);
    }
    put((i + 1) & 1, REV ? P - 2 - i : i + 1, a0 + (a1 + a2));
    lds_barrier();
  };
  {
    const float* X0 = c.X0 ? c.X0 + (size_t)bh * DD : nullptr;
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = X0 ? X0[(size_t)(r0 + 4 * g + e) * D + col] : 0.f;
    put(0, REV ? P - 1 : 0, x);
  }
  if (nst <= 0) return;
  ChainIn<D> p0, p1, p2;
  fetch(0, p0);
  fetch(1, p1);
  lds_barrier();
  for (int i = 0; i < nst; i += 3) {
    fetch(i + 2, p2);
    step(i, p0);
    if (i + 1 >= nst) break;
    fetch(i + 3, p0);
    step(i + 1, p1);
    if (i + 2 >= nst) break;
    fetch(i + 4, p1);
    step(i + 2, p2);
  }
}

// ------------------------------------------------------------ launch -------
static hipError_t set_lds(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int D>
hipError_t launch_fwd_summary(const FwdArgs& a, int nseg, hipStream_t st, Profiler* prof,
                              const char* name) {
  typedef FwdLds<T, D> Lz;
  constexpr size_t lds1 = Lz::sum_bytes, lds2 = Sum2Lds<T, D>::bytes;
  if constexpr (Sum2Lds<T, D>::fits) {
    hipError_t e = set_lds((const void*)gdn_fwd_summary2_kernel<T, D>, lds2);
    if (e != hipSuccess) return e;
    prof_begin(prof, name, st);
    hipLaunchKernelGGL((gdn_fwd_summary2_kernel<T, D>), dim3(a.B * a.H * nseg),
                       dim3(64 * fwd_nw<D>()), lds2, st, a, nseg);
    prof_end(prof, st);
  } else {
    hipError_t e = set_lds((const void*)gdn_fwd_summary_kernel<T, D>, lds1);
    if (e != hipSuccess) return e;
    prof_begin(prof, name, st);
    hipLaunchKernelGGL((gdn_fwd_summary_kernel<T, D>), dim3(a.B * a.H * nseg),
                       dim3(64 * fwd_nw<D>()), lds1, st, a, nseg);
    prof_end(prof, st);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_prep(const FwdArgs& a, hipStream_t st, Profiler* prof) {
  typedef PrepLds<T, D> Lz;
  hipError_t e = set_lds((const void*)gdn_prep_kernel<T, D>, Lz::bytes);
  if (e != hipSuccess) return e;
  prof_begin(prof, "gdn_prep", st);
  hipLaunchKernelGGL((gdn_prep_kernel<T, D>), dim3(a.B * a.H * a.nblk), dim3(256), Lz::bytes, st, a);
  prof_end(prof, st);
  return hipGetLastError();
}

template <int D, bool REV>
hipError_t launch_chain(const ChainArgs& c, hipStream_t st, Profiler* prof) {
  prof_begin(prof, REV ? "gdn_chain_bwd" : "gdn_chain_fwd", st);
  hipLaunchKernelGGL((gdn_chain_kernel<D, REV>), dim3(xcd_grid(c.BH, D / 16)), dim3(4 * D), 0, st,
                     c);
  prof_end(prof, st);
  return hipGetLastError();
}

// The fused out kernel in MODE: the two-blocks-in-flight form where its LDS
// layout fits, else the one-block form.
template <typename T, int D, int MODE>
static hipError_t launch_out(const FwdArgs& a, T* hst, hipStream_t st, Profiler* prof,
                             const char* name) {
  const dim3 grid(a.B * a.H * a.P), block(64 * fwd_nw<D>());
  hipError_t e;
  if (MODE != OUT_ONLY && (!hst || !a.vst)) return hipErrorInvalidValue;
  if constexpr (OutLds<T, D>::fits) {
    constexpr size_t ob = OutLds<T, D>::bytes;
    if ((e = set_lds((const void*)gdn_fwd_out2_kernel<T, D, MODE>, ob)) != hipSuccess) return e;
    prof_begin(prof, name, st);
    hipLaunchKernelGGL((gdn_fwd_out2_kernel<T, D, MODE>), grid, block, ob, st, a, hst);
  } else {
    constexpr size_t ob = FwdLds<T, D>::out_bytes;
    if ((e = set_lds((const void*)gdn_fwd_out_kernel<T, D, MODE>, ob)) != hipSuccess) return e;
    prof_begin(prof, name, st);
    hipLaunchKernelGGL((gdn_fwd_out_kernel<T, D, MODE>), grid, block, ob, st, a, hst);
  }
  prof_end(prof, st);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_states(const FwdArgs& a, void* hst, hipStream_t st, Profiler* prof) {
  return launch_out<T, D, STATES_ONLY>(a, reinterpret_cast<T*>(hst), st, prof, "gdn_fwd_states");
}

// hsave: when not null, every block's entry state is stored there and the
// segment maps M are computed for all P segments (a.MBseg then points into the
// caller's saved buffer), so that the backward can skip its recompute.
template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, void* hsave, int phase, hipStream_t st, Profiler* prof) {
  hipError_t e;
  const int BH = a.B * a.H;
  if (phase != PHASE_END) {  // Pre and the segment maps: independent of S_in
    if ((e = launch_prep<T, D>(a, st, prof)) != hipSuccess) return e;
    if (a.P > 1) {
      const int nseg = hsave ? a.P : a.P - 1;
      if ((e = launch_fwd_summary<T, D>(a, nseg, st, prof, "gdn_fwd_summary")) != hipSuccess)
        return e;
    }
    if (phase == PHASE_BEGIN) return hipSuccess;
  }
  if (a.P > 1) {
    ChainArgs c{a.S_in, a.Mseg, a.Nseg, const_cast<float*>(a.Sst), a.P, BH};
    if ((e = launch_chain<D, false>(c, st, prof)) != hipSuccess) return e;
  }
  if (hsave)
    return launch_out<T, D, OUT_AND_STATES>(a, reinterpret_cast<T*>(hsave), st, prof,
                                            "gdn_fwd_out_save");
  return launch_out<T, D, OUT_ONLY>(a, nullptr, st, prof, "gdn_fwd_out");
}

#define SF_INST(T, D)                                                                      \
  template hipError_t launch_fwd<T, D>(const FwdArgs&, void*, int, hipStream_t, Profiler*);  \
  template hipError_t launch_fwd_summary<T, D>(const FwdArgs&, int, hipStream_t, Profiler*, const char*); \
  template hipError_t launch_states<T, D>(const FwdArgs&, void*, hipStream_t, Profiler*);  \
  template hipError_t launch_prep<T, D>(const FwdArgs&, hipStream_t, Profiler*);
SF_INST(bf16, 128)
SF_INST(bf16, 64)
SF_INST(float, 128)
SF_INST(float, 64)
#undef SF_INST
template hipError_t launch_chain<128, false>(const ChainArgs&, hipStream_t, Profiler*);
template hipError_t launch_chain<64, false>(const ChainArgs&, hipStream_t, Profiler*);
template hipError_t launch_chain<128, true>(const ChainArgs&, hipStream_t, Profiler*);
template hipError_t launch_chain<64, true>(const ChainArgs&, hipStream_t, Profiler*);

}  // namespace sfgdn

// ------------------------------------------------------------ state copy ---
namespace sfgdn {
__global__ void copy_state_kernel(float* dst, const float* src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

// dst[0..n) = src (or zeros when src is null); a kernel rather than a memset
// or memcpy node so that callers may capture it in a graph.
hipError_t launch_copy_state(float* dst, const float* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

// ------------------------------------------------------------- casts -------
// Eight elements per thread; n is a multiple of 8 (a whole number of rows of
// width 64 or 128).  bf16 from fp32 rounds to nearest even.
__global__ void cast_to_f32_kernel(float* dst, const bf16* src, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const bf16x8 x = reinterpret_cast<const bf16x8*>(src)[i];
    f32x4* d = reinterpret_cast<f32x4*>(dst) + 2 * i;
    d[0] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    d[1] = f32x4{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
  }
}
__global__ void cast_to_bf16_kernel(bf16* dst, const float* src, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const f32x4 a = reinterpret_cast<const f32x4*>(src)[2 * i];
    const f32x4 b = reinterpret_cast<const f32x4*>(src)[2 * i + 1];
    reinterpret_cast<bf16x8*>(dst)[i] =
        bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
               (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
}
static unsigned cast_blocks(size_t n8) {
  size_t blocks = (n8 + 255) / 256;
  return (unsigned)(blocks > 4096 ? 4096 : blocks);
}
hipError_t launch_cast_to_f32(float* dst, const void* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cast_to_f32_kernel, dim3(cast_blocks(n / 8)), dim3(256), 0, st, dst,
                     reinterpret_cast<const bf16*>(src), n / 8);
  return hipGetLastError();
}
hipError_t launch_cast_to_bf16(void* dst, const float* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cast_to_bf16_kernel, dim3(cast_blocks(n / 8)), dim3(256), 0, st,
                     reinterpret_cast<bf16*>(dst), src, n / 8);
  return hipGetLastError();
}
}  // namespace sfgdn
