/*
 * sf_gdn.h -- C ABI of the MI355X (gfx950) library for one pipeline chunk of
 * the gated delta-rule recurrence (Gated DeltaNet), forward and backward.
 *
 * Source of the operation: "Pith review of StateFlow: Sequence Pipeline
 * Parallelism for Long-Context Modeling with Linear Recurrence"
 * (pith.science).
 *   - "What carries the argument": a sequence is split into chunks
 *     C_0 || ... || C_{N-1}; chunk C_i starts from its boundary state
 *     S_i^in and emits S_i^out; forward chaining S_{i+1}^in = S_i^out
 *     (Eq. 5) and backward chaining Sbar_i^out = Sbar_{i+1}^in (Eq. 7).
 *   - "Referee Report", major comment 1: the layer is the gated delta rule
 *     (Eq. (1)) with its auxiliary V_new path (Eq. (2)); the chunk backward
 *     must rebuild the chunk's state trajectory, which this library does by
 *     recomputing it from the chunk inputs.
 * Per (batch b, head h) sequence, with a d_v x d_k state S:
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 * alpha_t (decay, 0 < alpha <= 1) and beta_t (write strength) are scalars per
 * token and head; there is no query scaling and no normalisation inside.
 *
 * Layouts (all contiguous, row-major):
 *     q, k            [B, T, H, Dk]   dtype (bf16 or fp32)
 *     v, o, dO        [B, T, H, Dv]   dtype
 *     dq, dk, dv      like q, k, v    dtype
 *     alpha, beta     [B, T, H]       fp32
 *     dalpha, dbeta   [B, T, H]       fp32
 *     S_in, S_out, dS_out, dS_in   [B, H, Dv, Dk] fp32  (o_t = S_t q_t)
 * With B = 1 a pipeline chunk of a longer sequence is a pointer offset into
 * the sequence tensors (rows t0 .. t0+T-1), so chaining needs no copies.
 *
 * Ownership: the caller owns every buffer, including the workspace.  The
 * library allocates and frees no device memory and keeps no pointer after a
 * call returns.  All work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) with no host synchronisation; results are ready when the
 * stream reaches that point.  Calls are stateless and reentrant; results are
 * bitwise deterministic for a given shape and seg_blocks.
 *
 * Errors: arguments are checked on the host before anything is enqueued; on
 * failure nothing is enqueued and the status says why (details in
 * sf_last_error_message(), per thread).  No exception or abort crosses the
 * ABI.  Not checked (documented preconditions, checking would cost a pass over
 * HBM): 0 < alpha <= 1, finite inputs.  NaN inputs propagate.
 *
 * Supported: Dk == Dv in {64, 128} for bf16 and for fp32; any T >= 0 (a
 * partial last 64-token block is handled in the kernels).  The backward
 * workspace of fp32 at d = 128 includes 256 global tile areas of 132 KiB for
 * the gradient kernel (its tiles do not fit LDS at that size).  A bf16 chunk
 * of one 64-token block (T <= 64) is computed by the fp32 kernels on fp32
 * copies of its inputs, with o, dq, dk and dv rounded to bf16 at the end: its
 * workspaces include those copies and its saved buffer has the fp32 layout
 * (the workspace and saved-size queries account for both).
 */
#ifndef SF_GDN_H
#define SF_GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SF_OK = 0,
  SF_ERR_INVALID_ARG = 1,  /* null pointer, bad dimension, misalignment, aliasing */
  SF_ERR_UNSUPPORTED = 2,  /* valid request that the library does not implement */
  SF_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  SF_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} sf_status;

typedef enum { SF_DTYPE_F32 = 0, SF_DTYPE_BF16 = 1 } sf_dtype;

/* Problem description.  seg_blocks is the number of 64-token kernel blocks
 * per segment of the in-chunk parallel scan; 0 picks a default from the
 * shape.  Workspace sizes depend on it. */
typedef struct {
  int B, T, H, Dk, Dv;
  int dtype;       /* sf_dtype of q, k, v, o, dO, dq, dk, dv */
  int seg_blocks;  /* 0 = automatic */
} sf_gdn_shape;

/* The in-chunk parallel scan's plan for a shape: *seg_blocks kernel blocks
 * per segment and *segments segments (P = ceil(nblk / seg_blocks); 0 for an
 * empty chunk).  The segment-parallel form is the chunk chain of Eq. 5
 * applied inside the chunk.  With shape->seg_blocks = 0 the library picks
 * enough segments to occupy the GPU, but no fewer blocks per segment than
 * about sqrt(0.3 nblk).  Host only, no GPU call. */
sf_status sf_gdn_segment_plan(const sf_gdn_shape* shape, int* seg_blocks, int* segments);

/* Workspace bytes (256-byte aligned start required) for the calls below.
 * Returns SF_OK and writes *bytes, or an error for an unsupported shape. */
sf_status sf_gdn_chunk_fwd_workspace_size(const sf_gdn_shape* shape, size_t* bytes);
sf_status sf_gdn_chunk_bwd_workspace_size(const sf_gdn_shape* shape, size_t* bytes);

/* Forward of one chunk ("Fwd_i(S_i^in) -> S_i^out", Eq. 5 of the page).
 *   S_in   entry state, NULL means zeros.
 *   o      outputs (required when T > 0).
 *   S_out  exit state, may be NULL when not wanted.
 * Outputs must not overlap inputs or each other. */
sf_status sf_gdn_chunk_fwd(const sf_gdn_shape* shape, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S_in, void* o,
                           float* S_out, void* workspace, size_t ws_bytes, void* stream);

/* Backward of one chunk ("Bwd_i(Sbar_i^out) -> Sbar_i^in", Eq. 7 of the
 * page) of the loss L = <dO, o> + <dS_out, S_out>.  The inputs are the
 * forward's inputs (the chunk's state trajectory is recomputed from them);
 * dS_out NULL means zeros.  Writes dq, dk, dv (dtype), dalpha, dbeta (fp32,
 * gradients with respect to alpha and beta themselves) and dS_in (fp32, may
 * be NULL when not wanted).  dalpha keeps its accuracy down to the smallest
 * alpha: every term of d log alpha_t is formed with alpha_t as a factor
 * before the division by alpha_t (tested to alpha ~ 1e-15). */
sf_status sf_gdn_chunk_bwd(const sf_gdn_shape* shape, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S_in,
                           const void* dO, const float* dS_out, void* dq, void* dk, void* dv,
                           float* dalpha, float* dbeta, float* dS_in, void* workspace,
                           size_t ws_bytes, void* stream);

/* The forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what
 * sf_gdn_chunk_fwd computes, bit for bit, with the workspace taken from a
 * static device array of the library (64 MiB per GPU, held until the process
 * ends; its address is looked up once per device on the first call with that
 * device current).  It allocates and frees nothing.  A shape whose forward
 * workspace (sf_gdn_chunk_fwd_workspace_size) exceeds 64 MiB returns
 * SF_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * the same array, and nothing in it needs to start at any value: calls that
 * overlap in time on one GPU (two streams, two threads) race on it, so the
 * caller orders them (one stream, or events). */
sf_status sf_gdn_chunk_fwd_noalloc(const sf_gdn_shape* shape, const void* q, const void* k,
                                   const void* v, const float* alpha, const float* beta,
                                   const float* S_in, void* o, float* S_out, void* stream);

/* Saving forward and saved backward (no recompute of the forward scan).
 *
 * The backward above rebuilds the chunk's state trajectory from the inputs,
 * as the page's per-chunk activation release implies ("What carries the
 * argument"; Referee Report, major comment 1).  When memory allows keeping a
 * chunk's block states until its backward, sf_gdn_chunk_fwd_save also writes
 *   - the entry state of every 64-token block, B*H*ceil(T/64) states of
 *     Dv x Dk values in the q/k/v dtype (each state enters the backward's
 *     products in it), each in the library's internal tile order (the order
 *     in which its matrix-core accumulators hold it), not row-major
 *   - the segment transition maps of the in-chunk scan, row-major, fp32
 *     [B, H, P, Dk, Dk]
 *   - per block, T diag(beta) for T = (I + A)^{-1} of the block-local (WY/UT)
 *     form, [B, H, ceil(T/64), 64, 64] in the q/k/v dtype
 *   - per block, the auxiliary V^new = U - W S^T of the block-local form
 *     ("What carries the argument"; Referee Report, major comment 1: the
 *     backward needs the same V^new as the forward), 64 x Dv values in the
 *     q/k/v dtype, in the internal tile order
 * into the caller's `saved` buffer (size from sf_gdn_chunk_saved_size for
 * the same shape, 256-byte aligned; opaque otherwise), and
 * sf_gdn_chunk_bwd_saved computes the same gradients as sf_gdn_chunk_bwd from
 * it without S_in.  Results are bitwise those of the recompute path for the
 * same shape.  The workspaces are those of sf_gdn_chunk_fwd and
 * sf_gdn_chunk_bwd.  `saved` must not overlap any other argument. */
sf_status sf_gdn_chunk_saved_size(const sf_gdn_shape* shape, size_t* bytes);
sf_status sf_gdn_chunk_fwd_save(const sf_gdn_shape* shape, const void* q, const void* k,
                                const void* v, const float* alpha, const float* beta,
                                const float* S_in, void* o, float* S_out, void* saved,
                                size_t saved_bytes, void* workspace, size_t ws_bytes,
                                void* stream);
sf_status sf_gdn_chunk_bwd_saved(const sf_gdn_shape* shape, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const void* saved, size_t saved_bytes, const void* dO,
                                 const float* dS_out, void* dq, void* dk, void* dv, float* dalpha,
                                 float* dbeta, float* dS_in, void* workspace, size_t ws_bytes,
                                 void* stream);

/* Split-and-overlap of consecutive chunks on one GPU (the page's remedy for
 * the exposed state transition: kernels of other work fill the compute units
 * the state-transition kernels leave idle; Pith review of StateFlow, Figure 2
 * caption, and "Assumptions & free parameters", split fraction for overlap).
 * A chunk's call is cut into two launch groups:
 *   SF_PHASE_BEGIN  the launches that do not read S_in (forward: Pre and the
 *                   segment maps) or dS_out (backward: the segment
 *                   gradient maps from a zero exit gradient);
 *   SF_PHASE_END    the rest: the boundary-state chain and everything after
 *                   it; o, S_out (dq .. dS_in) are written here;
 *   SF_PHASE_ALL    both, which is the plain call.
 * BEGIN then END with the same arguments computes exactly what one ALL call
 * computes, bit for bit.  The caller keeps the workspace (and `saved`)
 * untouched between the two and orders END after BEGIN (same stream, or an
 * event).  With that, chunk i+1's BEGIN may run on another stream while chunk
 * i's END runs, each with its own workspace.  BEGIN does not read S_in,
 * dS_out, o, S_out or the gradient outputs, so they may still be in flight.
 * sf_gdn_chunk_fwd_split is sf_gdn_chunk_fwd (saved == NULL) or
 * sf_gdn_chunk_fwd_save; sf_gdn_chunk_bwd_saved_split is
 * sf_gdn_chunk_bwd_saved.  Arguments, layouts, ownership and errors are those
 * of the whole calls; an unknown phase is SF_ERR_INVALID_ARG. */
enum { SF_PHASE_ALL = 0, SF_PHASE_BEGIN = 1, SF_PHASE_END = 2 };
sf_status sf_gdn_chunk_fwd_split(const sf_gdn_shape* shape, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const float* S_in, void* o, float* S_out, void* saved,
                                 size_t saved_bytes, void* workspace, size_t ws_bytes, int phase,
                                 void* stream);
sf_status sf_gdn_chunk_bwd_saved_split(const sf_gdn_shape* shape, const void* q, const void* k,
                                       const void* v, const float* alpha, const float* beta,
                                       const void* saved, size_t saved_bytes, const void* dO,
                                       const float* dS_out, void* dq, void* dk, void* dv,
                                       float* dalpha, float* dbeta, float* dS_in, void* workspace,
                                       size_t ws_bytes, int phase, void* stream);

/* Short causal depthwise convolution of one chunk, with its boundary state
 * ("auxiliary local-convolution states" of a chunk: Pith review of StateFlow,
 * "What carries the argument"; their reconstruction in the chunked backward:
 * Referee Report, major comment 1).  The pages do not print the operation;
 * this is the usual causal depthwise 1-D convolution of width W along the
 * tokens, per channel c, over the chunk's inputs preceded by the previous
 * chunk's last W-1 inputs:
 *     xe = [conv_in (W-1 rows); x (T rows)]
 *     z_t = sum_{j<W} w[c][j] xe[t + W-1 - j][c]     (tap j = j tokens back)
 *     y_t = z_t (act = 0) or z_t * sigmoid(z_t) (act = 1, SiLU)
 *     conv_out = the last W-1 rows of xe (the next chunk's conv_in).
 * Chaining chunks through conv_out -> conv_in gives the unchunked result.
 * Layouts: x, y, dy, dx [B, T, C] and conv_in, conv_out, dconv_in, dconv_out
 * [B, W-1, C] in `dtype`; w, dw [C, W] fp32.  NULL conv_in / dconv_out mean
 * zeros; NULL conv_out / dconv_in mean not wanted.  1 <= W <= 8, C a
 * multiple of 8, pointers 16-byte aligned, outputs not overlapping inputs.
 * The backward writes dx, dconv_in and dw (the weight gradient summed over b
 * and t, not accumulated into dw's old contents) for the loss
 * <dy, y> + <dconv_out, conv_out>; its workspace (256-byte aligned) holds
 * per-run partial weight gradients, summed in a fixed order. */
typedef struct {
  int B, T, C, W;
  int dtype;  /* sf_dtype of x, y, conv states and their gradients */
  int act;    /* 0: none, 1: SiLU */
} sf_conv_shape;
sf_status sf_gdn_shortconv_fwd(const sf_conv_shape* shape, const void* x, const float* w,
                               const void* conv_in, void* y, void* conv_out, void* stream);
sf_status sf_gdn_shortconv_bwd_workspace_size(const sf_conv_shape* shape, size_t* bytes);
sf_status sf_gdn_shortconv_bwd(const sf_conv_shape* shape, const void* x, const float* w,
                               const void* conv_in, const void* dy, const void* dconv_out,
                               void* dx, float* dw, void* dconv_in, void* workspace,
                               size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* sf_status_string(int status);
/* Detail of the calling thread's last non-OK status (static until the next
 * failing call on this thread). */
const char* sf_last_error_message(void);
/* Library version string. */
const char* sf_gdn_version(void);

/* Per-kernel timing for measurement.  sf_gdn_profile_begin(capacity) makes
 * every following launch (up to `capacity`) record a HIP event pair on its
 * stream; sf_gdn_profile_end() waits for them and aggregates per kernel name.
 * Results stay readable until the next begin.  Process-wide; calls are
 * serialised internally. */
sf_status sf_gdn_profile_begin(int capacity);
sf_status sf_gdn_profile_end(void);
int sf_gdn_profile_kernel_count(void);
sf_status sf_gdn_profile_kernel(int index, const char** name, long long* launches,
                                double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SF_GDN_H */
