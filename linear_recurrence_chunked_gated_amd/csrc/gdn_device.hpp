// Device building blocks for the chunked gated delta rule on gfx950 (CDNA4).
//
// Conventions used by every kernel in this library:
//  * A kernel block is BLK = 64 consecutive tokens of one (batch, head)
//    sequence (the kernel-level blocks inside a pipeline chunk, Pith review of
//    StateFlow, "Assumptions", domain assumption on kernel-level chunking).
//  * Matrix products run on MFMA 16x16 tiles: v_mfma_f32_16x16x32_bf16 for
//    bf16 operands and v_mfma_f32_16x16x4_f32 for fp32 operands, always
//    accumulating in fp32.  Products are written C[m][n] += sum_k A[m][k] B[n][k].
//  * An operand fragment gives lane l = 16 g + i row i of the operand (its m
//    or n index) and, per instruction, KPL contraction elements whose k index
//    depends on g.  Two k orders are used, and both operands of one product
//    must use the same order:
//      STD   k = 8 g + j                                 (bf16, j = 0..7)
//            k = g                                       (fp32)
//      PERM  k = 4 g + (j & 3) + 16 (j >> 2)             (bf16)
//            k = 16 (s / 4) + 4 g + (s % 4) at step s    (fp32)
//    PERM is the order in which an accumulator tile already holds its values
//    (lane l owns C[m = 4 g + e][n = i]), so an accumulator can be fed back as
//    an operand whose rows are its n index and whose contraction index is its
//    m index, without leaving registers.
//  * Operands in LDS are row-major tiles.  bf16 tiles have unpadded rows of
//    128 or 256 bytes, stored swizzled (see lds_sw); fp32 tiles are padded by
//    16 bytes per row.  A tile stored as X[k][n] (contraction index on rows)
//    is read as an operand with rows n through the gfx950 transpose read
//    ds_read_b64_tr_b16: within each 16-lane group, input lane m addresses
//    row m / 4, columns 4 (m % 4) .. +3, and output lane i receives column i
//    of those 4 rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfgdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BLK = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Workgroup barrier for LDS hand-offs.  It waits only for this wave's LDS
// (and scalar) operations; outstanding global loads and stores stay in
// flight.  (__syncthreads() would also drain vmcnt.)
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// A barrier after which the other waves of the workgroup also see this wave's
// global stores: the stores are complete (vmcnt) and a workgroup's waves share
// one compute unit and its vector L1.  For tiles kept in a per-workgroup
// global area instead of LDS.
__device__ __forceinline__ void full_barrier() {
  __asm__ __volatile__("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void vm_wait() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cross-lane sums without an LDS round trip: DPP within a 16-lane row, and
// across rows the gfx950 lane swaps (v_permlane16/32_swap) or lane reads.
// dpp_f: lanes whose DPP source lies outside their row receive 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// sum over the 16 lanes of a row (quad_perm [1,0,3,2], [2,3,0,1], half-row
// mirror, row mirror); every lane of the row ends with the total
__device__ __forceinline__ float sum_row16(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}
// sum over the 4 rows (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum over the 64 lanes of the wave, in every lane
__device__ __forceinline__ float wave_sum(float x) { return sum_rows4(sum_row16(x)); }
// Inclusive prefix sum over lanes 0..l: row shifts right by 1, 2, 4, 8 within
// each row, then the totals of the rows below (lanes 15, 31, 47).
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  x += dpp_f<0x118>(x);
  const float r0 = lane_f(x, 15), r1 = lane_f(x, 31), r2 = lane_f(x, 47);
  const int row = lane_id() >> 4;
  return x + (row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2);
}
// Inclusive suffix sum over lanes l..63: row shifts left by 1, 2, 4, 8, then
// the totals of the rows above (lanes 16, 32, 48).
__device__ __forceinline__ float wave_suffix_sum(float x) {
  x += dpp_f<0x101>(x);
  x += dpp_f<0x102>(x);
  x += dpp_f<0x104>(x);
  x += dpp_f<0x108>(x);
  const float r1 = lane_f(x, 16), r2 = lane_f(x, 32), r3 = lane_f(x, 48);
  const int row = lane_id() >> 4;
  return x + (row == 3 ? 0.f : row == 2 ? r3 : row == 1 ? r2 + r3 : r1 + (r2 + r3));
}

enum KOrder { STD = 0, PERM = 1 };

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  typedef bf16x8 frag;
  static constexpr int KSTEP = 32;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  typedef float frag;
  static constexpr int KSTEP = 4;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <typename T> struct Lay {
  static constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  // Row padding (elements): none for the swizzled bf16 tiles, 16 bytes for
  // fp32 tiles (so that 16 rows of a 4-byte fragment read hit distinct banks).
  static constexpr int PAD = sizeof(T) == 2 ? 0 : VEC;
  static constexpr int PADC = PAD;
  // Padded bf16 rows, for kernels that keep them instead of the swizzle:
  // 16 bytes per row (32 for 64-wide tiles that are mostly read by rows).
  static constexpr int PADX = VEC;
  static constexpr int PADXC = sizeof(T) == 2 ? 2 * VEC : VEC;
  typedef T pack4 __attribute__((ext_vector_type(4)));
};

// LDS region offsets: swizzled tiles start on 4 KiB boundaries (16 rows of
// 256 bytes), so that a tile's row index is in the address bits lds_sw reads.
constexpr size_t lds_align(size_t x) { return (x + 4095) / 4096 * 4096; }

// The LDS position of element address p of a row-major bf16 tile with ld
// elements per row.  Rows of 256 bytes (16 chunks of 16 bytes) store chunk c
// of row r at c ^ (r & 15), rows of 128 bytes at c ^ ((r >> 1) & 7); any other
// row length, and fp32 tiles, are stored as addressed (padded rows).
// Measured on gfx950 with 8 waves (cycles per wave instruction), these masks
// put every access form of the kernels at its conflict-free cost: 16-byte row
// reads of 16 rows x 4 chunks 4.4 (8.1 with 272-byte padded rows, 8.0 with
// 144-byte ones), 8-byte row-pair reads 5.5, transpose reads 4.2, 8-byte
// transposed stores 8 and 2-byte stores 4, none worse than padded rows.
// The mask is a function of the address alone (tiles are 4 KiB aligned), so
// it is applied to final element addresses, on the 32-bit LDS address.  A
// kernel that keeps padded rows (ld of any other length) gets p unchanged.
template <typename T>
__device__ __forceinline__ T* lds_sw(T* p, int ld) {
  const int rowb = ld * (int)sizeof(T);
  if (sizeof(T) != 2 || (rowb != 256 && rowb != 128)) return p;
  typedef __attribute__((address_space(3))) T lds_t;
  const unsigned a = (unsigned)(size_t)(lds_t*)p;  // the 32-bit LDS address
  const unsigned b = a ^ ((a >> 4) & (rowb == 256 ? 0xF0u : 0x70u));
  return (T*)(lds_t*)(size_t)b;
}
template <typename T>
__device__ __forceinline__ const T* lds_sw(const T* p, int ld) {
  return lds_sw(const_cast<T*>(p), ld);
}

// ---------------------------------------------------------------- frags ----
// Operand rows from a row-major LDS tile: p points at the fragment's row 0
// (the operand's m or n index), k runs along the row.  s is the k-step.
template <typename T, int KO> __device__ __forceinline__ typename Mma<T>::frag
frag_row(const T* p, int ld, int s);

template <> __device__ __forceinline__ bf16x8 frag_row<bf16, STD>(const bf16* p, int ld, int s) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(lds_sw(p + (l & 15) * ld + 32 * s + 8 * (l >> 4), ld));
}
template <> __device__ __forceinline__ bf16x8 frag_row<bf16, PERM>(const bf16* p, int ld, int s) {
  const int l = lane_id();
  const bf16* q = p + (l & 15) * ld + 32 * s + 4 * (l >> 4);
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(lds_sw(q, ld));
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(lds_sw(q + 16, ld));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <> __device__ __forceinline__ float frag_row<float, STD>(const float* p, int ld, int s) {
  const int l = lane_id();
  return p[(l & 15) * ld + 4 * s + (l >> 4)];
}
template <> __device__ __forceinline__ float frag_row<float, PERM>(const float* p, int ld, int s) {
  const int l = lane_id();
  return p[(l & 15) * ld + 16 * (s >> 2) + 4 * (l >> 4) + (s & 3)];
}

// Operand rows n0.. from a tile stored X[k][n] (k on rows): the operand is
// X^T.  p points at X[0][n0].
template <typename T, int KO> __device__ __forceinline__ typename Mma<T>::frag
frag_tr(const T* p, int ld, int s);

__device__ __forceinline__ bf16x4 ds_tr4(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}
// rows k0 .. k0+3 of X, columns n0 .. n0+15, delivered transposed.
__device__ __forceinline__ bf16x4 tr_rows4(const bf16* p, int ld, int k0) {
  const int i = lane_id() & 15;
  return ds_tr4(lds_sw(p + (k0 + (i >> 2)) * ld + 4 * (i & 3), ld));
}
template <> __device__ __forceinline__ bf16x8 frag_tr<bf16, STD>(const bf16* p, int ld, int s) {
  const int g = lane_id() >> 4;
  const bf16x4 lo = tr_rows4(p, ld, 32 * s + 8 * g);
  const bf16x4 hi = tr_rows4(p, ld, 32 * s + 8 * g + 4);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <> __device__ __forceinline__ bf16x8 frag_tr<bf16, PERM>(const bf16* p, int ld, int s) {
  const int g = lane_id() >> 4;
  const bf16x4 lo = tr_rows4(p, ld, 32 * s + 4 * g);
  const bf16x4 hi = tr_rows4(p, ld, 32 * s + 16 + 4 * g);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <> __device__ __forceinline__ float frag_tr<float, STD>(const float* p, int ld, int s) {
  const int l = lane_id();
  return p[(4 * s + (l >> 4)) * ld + (l & 15)];
}
template <> __device__ __forceinline__ float frag_tr<float, PERM>(const float* p, int ld, int s) {
  const int l = lane_id();
  return p[(16 * (s >> 2) + 4 * (l >> 4) + (s & 3)) * ld + (l & 15)];
}

// Operand from accumulator tiles acc[0 .. ] whose m index is the contraction
// index (PERM order), each element scaled by sc[m-tile][e] when given.
template <typename T> struct AccFrag;
template <> struct AccFrag<bf16> {
  // k-step s uses tiles 2s and 2s+1
  __device__ static __forceinline__ bf16x8 get(const f32x4* t, int s) {
    const f32x4 a = t[2 * s], b = t[2 * s + 1];
    return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                  (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
  __device__ static __forceinline__ bf16x8 get_scaled(const f32x4* t, const f32x4* sc, int s) {
    const f32x4 a = t[2 * s] * sc[2 * s], b = t[2 * s + 1] * sc[2 * s + 1];
    return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                  (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
};
template <> struct AccFrag<float> {
  __device__ static __forceinline__ float get(const f32x4* t, int s) { return t[s >> 2][s & 3]; }
  __device__ static __forceinline__ float get_scaled(const f32x4* t, const f32x4* sc, int s) {
    return t[s >> 2][s & 3] * sc[s >> 2][s & 3];
  }
};

template <int MI, int NJ>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MI][NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int MI, int NJ>
__device__ __forceinline__ void scale_acc(f32x4 (&acc)[MI][NJ], float s) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] *= s;
}

// fp32 product with a row-major right operand: acc += A[m][:K] * B[:K][n].
// Used by the small unit-lower solve.
template <int K>
__device__ __forceinline__ void gemm_nn_f32(f32x4& acc, const float* A, int lda, const float* B,
                                            int ldb) {
  const int lane = lane_id();
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int k = 0; k < K; k += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k + kq], B[(k + kq) * ldb + r], acc, 0,
                                               0, 0);
}

__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

template <typename T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// Four consecutive elements as fp32.
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Per-block states (and state gradients) in HBM, D x D values per block, in
// the order the MFMA accumulators hold them: the 16 x D tile of wave w
// (rows 16 w ..), then, per lane, 16-byte vectors of the lane's
// accumulator entries.  Lane l = i + 16 g holds, for each 16 x 16 tile a,
// rows 16 w + i and columns 16 a + 4 g .. + 3; vector v packs tiles
// v * TPV .. + TPV - 1.  Every store and load of a state is then one
// contiguous 1 KiB per wave instruction.
template <typename T, int D> struct StateTiles {
  static constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int TPV = E / 4;              // 16 x 16 tiles per vector
  static constexpr int NV = D / 16 / TPV;        // vectors per lane
  static_assert(TPV >= 1 && NV * TPV == D / 16, "tile packing");
  __device__ static __forceinline__ size_t off(int w, int lane, int v) {
    return (size_t)w * 16 * D + (size_t)v * 64 * E + (size_t)lane * E;
  }
  __device__ static __forceinline__ void store(T* blockbase, int w, int lane, const f32x4* x) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (TPV == 2) {
        const f32x4 a = x[2 * v], b = x[2 * v + 1];
        const bf16x8 h = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                          (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
        *reinterpret_cast<bf16x8*>(blockbase + off(w, lane, v)) = h;
      } else {
        *reinterpret_cast<f32x4*>(blockbase + off(w, lane, v)) = x[v];
      }
    }
  }
  __device__ static __forceinline__ void load(const T* blockbase, int w, int lane, f32x4* x) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (TPV == 2) {
        const bf16x8 h = *reinterpret_cast<const bf16x8*>(blockbase + off(w, lane, v));
        x[2 * v] = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
        x[2 * v + 1] = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
      } else {
        x[v] = *reinterpret_cast<const f32x4*>(blockbase + off(w, lane, v));
      }
    }
  }
  // The same in two steps: the loads, then (once their data is needed) the
  // conversion, so that the loads can stay in flight meanwhile.
  __device__ static __forceinline__ void load_raw(const T* blockbase, int w, int lane,
                                                  uint4 (&r)[NV]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) r[v] = *reinterpret_cast<const uint4*>(blockbase + off(w, lane, v));
  }
  __device__ static __forceinline__ void unpack(const uint4 (&r)[NV], f32x4* x) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (TPV == 2) {
        const bf16x8 h = __builtin_bit_cast(bf16x8, r[v]);
        x[2 * v] = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
        x[2 * v + 1] = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
      } else {
        x[v] = __builtin_bit_cast(f32x4, r[v]);
      }
    }
  }
};

// LDS tile dst[n][m..m+3] = scale * acc for the tile at (m0, n0).
template <typename T>
__device__ __forceinline__ void store_tile_T(const f32x4& acc, T* dst, int ld, int m0, int n0,
                                             float scale = 1.f) {
  const int lane = lane_id();
  const int m = m0 + 4 * (lane >> 4), n = n0 + (lane & 15);
  st4(lds_sw(dst + n * ld + m, ld), scale * acc[0], scale * acc[1], scale * acc[2],
      scale * acc[3]);
}

// LDS tile dst[m + e][n] = scale * acc[e].
template <typename T>
__device__ __forceinline__ void store_tile_N(const f32x4& acc, T* dst, int ld, int m0, int n0,
                                             float scale = 1.f) {
  const int lane = lane_id();
  const int m = m0 + 4 * (lane >> 4), n = n0 + (lane & 15);
#pragma unroll
  for (int e = 0; e < 4; ++e) *lds_sw(dst + (m + e) * ld + n, ld) = from_f<T>(scale * acc[e]);
}

// ---------------------------------------------------------------------------
// Moving 64-row tiles from HBM to LDS.  A tile is BLK rows of D elements of
// type T; each of NT threads moves NCH 16-byte chunks, consecutive threads
// covering consecutive chunks of a row.  Loads are unconditional (rows past
// the end of the sequence re-read its last row, which is in bounds) and the
// tail rows are zeroed when the tile is written to LDS, so no branch sits
// between a load and its use.
// ---------------------------------------------------------------------------
template <typename T, int D, int NT> struct Tile {
  static constexpr int VEC = Lay<T>::VEC;
  static constexpr int CPR = D / VEC;
  static constexpr int NCH = BLK * CPR / NT;
  static_assert((BLK * CPR) % NT == 0, "tile must split evenly over the workgroup");

  __device__ static __forceinline__ void load(uint4 (&r)[NCH], const T* g, size_t row_stride,
                                              int nvalid) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = threadIdx.x + NT * it;
      const int row = min(c / CPR, nvalid - 1), ch = c % CPR;
      r[it] = *reinterpret_cast<const uint4*>(g + (size_t)row * row_stride + ch * VEC);
    }
  }

  __device__ static __forceinline__ void to_lds(const uint4 (&r)[NCH], T* s, int ld, int nvalid) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = threadIdx.x + NT * it;
      const int row = c / CPR, ch = c % CPR;
      const bool ok = row < nvalid;
      uint4 v = r[it];
      v.x = ok ? v.x : 0u;
      v.y = ok ? v.y : 0u;
      v.z = ok ? v.z : 0u;
      v.w = ok ? v.w : 0u;
      *reinterpret_cast<uint4*>(lds_sw(s + row * ld + ch * VEC, ld)) = v;
    }
  }
};

}  // namespace sfgdn
