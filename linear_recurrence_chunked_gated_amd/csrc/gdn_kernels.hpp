// Kernel argument blocks and launch entry points shared by the forward and
// backward translation units and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "gdn_block.hpp"

namespace sfgdn {

// One chunk call.  Token-major tensors are [B, T, H, D]; gates [B, T, H];
// states [B, H, D, D] fp32 ([dv][dk] row-major).  The chunk's nblk blocks are
// split into P segments of L blocks (the last one may be shorter).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S_in;   // may be null (zeros)
  void* o;             // may be null for state-only passes
  float* S_out;        // may be null
  int B, T, H;
  int nblk, L, P;
  // workspace
  float* Mseg;         // [B*H][P][D][D]  segment transition maps M (S' = S M + N), transposed:
                       //                  MT[n][k] = M[k][n], the forward chain's operand
  float* MBseg;        // [B*H][P][D][D]  the same maps row-major (the backward chain's), or null
  float* Nseg;         // [B*H][P][D][D]  segment zero-entry exit states
  const float* Sst;    // [B*H][sst_P][D][D] segment entry states (S_in when P == 1)
  int sst_P;
  void* tw;            // [B*H][nblk][64][64] per-block Tpp (operand type), by the Pre kernel
  void* vst;           // [B*H][nblk][64 x D] per-block Vn (operand type, in the order of
                       // StateTiles<T, 64>: wave w's 64 x 16 slice, dv-tile w), written by
                       // the state-storing forward and read by the gradient kernel
};

// One boundary-state chain over the P segments of each sequence (see
// gdn_chain_kernel): entry X0 (null = zeros), per-segment B_j^T and C_j,
// all P states out.
struct ChainArgs {
  const float* X0;
  const float* Bt;
  const float* C;
  float* out;
  int P;
  int BH;
};

// Workgroups are handed to the 8 XCDs round-robin (workgroup i runs on XCD
// i % 8), and each XCD has its own L2.  The chain kernels run RT workgroups
// per sequence, all reading the same segment maps, so they are placed on one
// XCD: workgroup i takes sequence bh (>= BH for padding workgroups, which
// exit) and row tile r.
constexpr int kXcds = 8;
__host__ __device__ inline void xcd_seq_tile(int i, int RT, int& bh, int& r) {
  const int x = i % kXcds, s = i / kXcds;
  bh = x + kXcds * (s / RT);
  r = s % RT;
}
inline int xcd_grid(int BH, int RT) { return (BH + kXcds - 1) / kXcds * kXcds * RT; }

struct BwdArgs {
  FwdArgs f;            // inputs, plan and forward workspace (o, S_out unused)
  const void* dO;       // [B, T, H, D]
  const float* dS_out;  // may be null (zeros)
  void* dq;
  void* dk;
  void* dv;
  float* dalpha;
  float* dbeta;
  float* dS_in;         // may be null
  // workspace
  float* NBseg;         // [B*H][P][D][D] segment state-gradient maps from a zero exit gradient
  float* dSend;         // [B*H][P][D][D] state gradient at each segment's exit
  void* hst;            // [B*H][nblk][D][D] block entry states (state storage type)
  void* dhst;           // [B*H][nblk][D][D] gradient wrt each block's exit state
  void* far;            // the gradient kernel's global tile areas (see bwd_far_bytes), or null
};

// Where the gradient kernel's input tiles do not fit its LDS plan (fp32 at
// d = 128) they live in global areas, one per workgroup, and a grid of at
// most kFarGroups workgroups (one per compute unit) strides over the blocks.
constexpr int kFarGroups = 256;
// Bytes of those areas for the operand type and head size (0: tiles in LDS).
size_t bwd_far_bytes(bool f32, int D);

// Short causal convolution of one chunk (see gdn_conv.hip).  Token tensors
// [B, T, C] and boundary states [B, W-1, C] in the operand type; weights and
// their gradient [C, W] fp32.  Null conv states mean zeros / not wanted.
struct ConvArgs {
  const void* x;
  const float* w;
  const void* cin;
  void* y;
  void* cout;
  const void* dy;
  const void* dcout;
  void* dx;
  float* dw;
  void* dcin;
  int B, T, C, W, act;
};

// Optional per-launch event timing (see sf_gdn_profile_* in the C ABI).
struct Profiler;
void prof_begin(Profiler* p, const char* name, hipStream_t st);
void prof_end(Profiler* p, hipStream_t st);

// A chunk's work in two parts, so that a caller can overlap the part that
// does not read the boundary state of one chunk with the rest of another:
// PHASE_BEGIN runs the launches that do not read S_in (dS_out), PHASE_END the
// others; PHASE_ALL both, in order.
enum { PHASE_ALL = 0, PHASE_BEGIN = 1, PHASE_END = 2 };

// hsave: optional per-block entry-state output (see launch_fwd).
template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, void* hsave, int phase, hipStream_t st, Profiler* prof);
// Pieces of the forward reused by the backward.
template <typename T, int D>
hipError_t launch_fwd_summary(const FwdArgs& a, int nseg, hipStream_t st, Profiler* prof,
                              const char* name);
template <typename T, int D>
hipError_t launch_prep(const FwdArgs& a, hipStream_t st, Profiler* prof);
template <int D, bool REV>
hipError_t launch_chain(const ChainArgs& c, hipStream_t st, Profiler* prof);
template <typename T, int D>
// Every block's entry state into hst and its Vn into a.vst.
hipError_t launch_states(const FwdArgs& a, void* hst, hipStream_t st, Profiler* prof);
// saved: a.hst already holds every block's entry state, a.f.MBseg every
// segment's map, a.f.tw every block's Tpp and a.f.vst every block's Vn (from
// a saving forward), so the forward recompute is skipped; otherwise the
// recompute writes the entry states and Vn into a.hst and a.f.vst.
// phase: PHASE_BEGIN and PHASE_END only with saved.
template <typename T, int D>
hipError_t launch_bwd(const BwdArgs& a, bool saved, int phase, hipStream_t st, Profiler* prof);
// Short convolution: GR tokens per backward run; dwp holds the B * ceil(T/GR)
// partial weight gradients [C][W] fp32 and room for their group sums.
template <typename T>
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st, Profiler* prof);
template <typename T>
hipError_t launch_conv_bwd(const ConvArgs& a, int GR, float* dwp, hipStream_t st, Profiler* prof);

}  // namespace sfgdn
