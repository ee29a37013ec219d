// Device building blocks for the chunked gated delta rule on gfx950 (CDNA4).
//
// Conventions used by every kernel in this library:
//  * A kernel block is BLK = 64 consecutive tokens of one (batch, head)
//    sequence ("kernel-level blocks b_{i,j} inside a pipeline chunk", Pith
//    review of StateFlow, "Assumptions", domain assumption on kernel-level
//    chunking).
//  * Workgroups have NWAVE = 8 wave64s.  Matrix products run on MFMA
//    16x16 tiles: v_mfma_f32_16x16x32_bf16 for bf16 operands and
//    v_mfma_f32_16x16x4_f32 for fp32 operands, always accumulating in fp32.
//  * Operands live in LDS as row-major tiles whose rows are contiguous along
//    the contraction index ("NT" form: C[m][n] += sum_k A[m][k] B[n][k]).
//    Rows are padded by 16 bytes to spread LDS banks.
//  * An accumulator tile holds C[m][n] with m = 4*(lane/16) + e (e = 0..3)
//    and n = lane % 16.  Storing it "transposed" (dst[n][m..m+3]) is one
//    vector write per lane; storing it as-is is four scalar writes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfgdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BLK = 64;
constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  typedef bf16x8 frag;
  static constexpr int KSTEP = 32;  // contraction depth of one instruction
  static constexpr int KPL = 8;     // contraction elements held per lane
  __device__ static __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  typedef float frag;
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  __device__ static __forceinline__ frag load(const float* p) { return *p; }
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Elements per 16-byte chunk and padded leading dimensions.
template <typename T> struct Lay {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int PAD = VEC;
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

// acc[i][j] += A[16i + m][:K] . B[16j + n][:K]; A and B point at the wave's
// first row, both K-contiguous.
template <typename T, int MI, int NJ, int K>
__device__ __forceinline__ void gemm_nt(f32x4 (&acc)[MI][NJ], const T* A, int lda,
                                        const T* B, int ldb) {
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * Mma<T>::KPL;
#pragma unroll
  for (int k = 0; k < K; k += Mma<T>::KSTEP) {
    typename Mma<T>::frag a[MI], b[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = Mma<T>::load(A + (16 * i + r) * lda + k + kq);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = Mma<T>::load(B + (16 * j + r) * ldb + k + kq);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = Mma<T>::mma(a[i], b[j], acc[i][j]);
  }
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

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// dst[n][m..m+3] = scale * acc for the tile at (m0, n0).
template <typename T>
__device__ __forceinline__ void store_tile_T(const f32x4& acc, T* dst, int ld, int m0, int n0,
                                             float scale = 1.f) {
  const int lane = lane_id();
  const int m = m0 + 4 * (lane >> 4), n = n0 + (lane & 15);
  st4(dst + n * ld + m, scale * acc[0], scale * acc[1], scale * acc[2], scale * acc[3]);
}

// dst[m + e][n] = scale * acc[e].
template <typename T>
__device__ __forceinline__ void store_tile_N(const f32x4& acc, T* dst, int ld, int m0, int n0,
                                             float scale = 1.f) {
  const int lane = lane_id();
  const int m = m0 + 4 * (lane >> 4), n = n0 + (lane & 15);
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[(m + e) * ld + n] = from_f<T>(scale * acc[e]);
}

// ---------------------------------------------------------------------------
// Moving 64-row tiles between HBM and LDS.  A tile is BLK rows of D elements
// of type T; each thread moves NCH 16-byte chunks.  Within a group of 16 rows
// the chunk index runs fastest over rows, so a wave touches 16 rows x 4
// chunks (64 contiguous bytes per row) and the transposed LDS scatter hits
// 16 consecutive columns.
// ---------------------------------------------------------------------------
template <typename T, int D> struct Tile {
  static constexpr int VEC = Lay<T>::VEC;
  static constexpr int CPR = D / VEC;                 // chunks per row
  static constexpr int NCHUNK = BLK * CPR;
  static constexpr int NCH = NCHUNK / NTHR;           // chunks per thread
  static_assert(NCHUNK % NTHR == 0, "tile must split evenly over the workgroup");

  __device__ static __forceinline__ void coords(int c, int& row, int& ch) {
    const int slot = c % (16 * CPR);
    row = 16 * (c / (16 * CPR)) + (slot & 15);
    ch = slot >> 4;
  }

  // Rows >= nvalid read as zero.  row_stride is in elements.
  __device__ static __forceinline__ void load(uint4 (&r)[NCH], const T* g, size_t row_stride,
                                              int nvalid) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      int row, ch;
      coords(threadIdx.x + NTHR * it, row, ch);
      if (row < nvalid)
        r[it] = *reinterpret_cast<const uint4*>(g + (size_t)row * row_stride + ch * VEC);
      else
        r[it] = uint4{0u, 0u, 0u, 0u};
    }
  }

  __device__ static __forceinline__ void to_lds(const uint4 (&r)[NCH], T* s, int ld) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      int row, ch;
      coords(threadIdx.x + NTHR * it, row, ch);
      *reinterpret_cast<uint4*>(s + row * ld + ch * VEC) = r[it];
    }
  }

  // sT[col][row] = tile[row][col]
  __device__ static __forceinline__ void to_lds_T(const uint4 (&r)[NCH], T* sT, int ldT) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      int row, ch;
      coords(threadIdx.x + NTHR * it, row, ch);
      const T* e = reinterpret_cast<const T*>(&r[it]);
#pragma unroll
      for (int x = 0; x < VEC; ++x) sT[(ch * VEC + x) * ldT + row] = e[x];
    }
  }

  // Row-major LDS tile -> HBM rows < nvalid, coalesced along rows.
  __device__ static __forceinline__ void store(const T* s, int ld, T* g, size_t row_stride,
                                               int nvalid) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = threadIdx.x + NTHR * it;
      const int row = c / CPR, ch = c % CPR;
      if (row < nvalid)
        *reinterpret_cast<uint4*>(g + (size_t)row * row_stride + ch * VEC) =
            *reinterpret_cast<const uint4*>(s + row * ld + ch * VEC);
    }
  }
};

}  // namespace sfgdn
