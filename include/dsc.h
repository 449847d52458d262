/*
 * dsc.h -- C ABI of the dynamic short convolution library (libdsc.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation ("Dynamic Short Convolutions Improve Transformers",
 * gist.science technical summary, Methodology, "mechanism"): for token n of
 * a sequence and channel d,
 *
 *     y[n,d] = rho * x[n,d] + sum_{k=0}^{W-1} w(n)_{d,k} * x[n-k,d]
 *
 * with a filter w(n) that belongs to the token.  x[n-k] is zero when n-k lies
 * before the first token of n's sequence (causal zero padding; the authors'
 * thread on digg.com describes the static short convolution being
 * generalised as causal).  rho in {0,1} selects the residual placement
 * X = X + dynamicShortConv(X) (same summary, Methodology, "placement").
 * Two filter parametrisations (Methodology, "parametrization"):
 *   - head-wise tying: one W-tap filter per token shared by H consecutive
 *     channels, w(n)_{d,k} = w[n, d/H, k];
 *   - low rank R: w(n)_{d,k} = sum_r z[n,r] * U[r, d*W + k], generated on
 *     chip and never written to memory (Efficient training implementation,
 *     fused low-rank kernel).
 * The backward entry points return the gradients of L = <dy, y>.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   stream      a hipStream_t passed as void*; NULL selects the null stream.
 *               Every call is asynchronous on that stream; device faults
 *               surface at the caller's next synchronisation.
 *   dtype       DSC_FP32 or DSC_BF16: the element type of every activation,
 *               filter and z/U tensor of the call (dU and dc are always
 *               fp32).  Arithmetic is fp32 (fused multiply-add) and each
 *               output is rounded once, to nearest even, to its storage type.
 *   B, T, D     batch, tokens per row and channels; tensors named (B,T,D)
 *               are dense row-major with channels innermost.  B or T may
 *               be 0 (an empty batch): the call then computes nothing
 *               except that the low-rank and static backward zero-fill dU
 *               and dc, and the pointers of tensors without elements may
 *               be NULL.  Decoding calls take B sequences of one token.
 *   W           taps, 1..8.
 *   cu_seqlens  NULL with n_seqs == 0: each of the B rows is one sequence.
 *               Otherwise a DEVICE pointer to int32[n_seqs+1] strictly
 *               increasing offsets on the flattened N = B*T token axis,
 *               cu_seqlens[0] = 0 and cu_seqlens[n_seqs] = N; sequences are
 *               defined by these offsets alone and may cross row boundaries.
 *               The contents are not validated (a malformed array gives
 *               undefined results).
 *   residual    0 or 1 (rho above).
 *   pointers    DEVICE pointers, each 16-byte aligned (the int32 arrays
 *               cu_seqlens and positions: 4-byte).  The caller owns all
 *               memory; the library allocates nothing, keeps no state and
 *               is thread-safe.  Inputs are never written.  Every output is
 *               fully overwritten (nothing accumulates into it), except the
 *               decoding state, which is updated in place.  No output may
 *               overlap an input or another output (so y = x in place is
 *               rejected).
 *
 * Errors: each entry point checks every host-checkable precondition first
 * and returns a status without making any HIP call when one fails; a failed
 * kernel launch returns DSC_ERR_HIP.  dsc_last_error() describes the most
 * recent failure of the calling thread.
 */
#ifndef DSC_H
#define DSC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSC_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define DSC_API __attribute__((visibility("default")))
#else
#define DSC_API
#endif

typedef enum dsc_dtype { DSC_FP32 = 0, DSC_BF16 = 1 } dsc_dtype;

typedef enum dsc_status {
    DSC_SUCCESS = 0,
    DSC_ERR_NULL = 1,        /* a required pointer is NULL                          */
    DSC_ERR_SHAPE = 2,       /* a size is out of range or inconsistent              */
    DSC_ERR_UNSUPPORTED = 3, /* valid shape this build does not implement           */
    DSC_ERR_ALIGNMENT = 4,   /* a pointer is not 16-byte aligned                    */
    DSC_ERR_ALIAS = 5,       /* an output overlaps an input or another output       */
    DSC_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required          */
    DSC_ERR_HIP = 7          /* a HIP call or kernel launch failed                  */
} dsc_status;

/*
 * Head-wise forward.  Methodology, "mechanism" and "parametrization (2)":
 * y[n,d] = rho*x[n,d] + sum_{k<W, n-k in n's sequence} w[n, d/H, k] * x[n-k,d].
 *
 *   x  (B,T,D) dtype, in.      w  (B,T,D/H,W) dtype, in (tap innermost).
 *   y  (B,T,D) dtype, out.
 *   H  channels per shared filter: any H >= 1 with D % H == 0 (the
 *      pages' "H consecutive channels" has no other restriction).  Groups
 *      that a 16-byte channel vector (8 bf16 / 4 fp32) holds whole, or that
 *      cover at most 64 whole vectors, run the streaming kernels; every other
 *      H (e.g. 3, 5, 6, 12, or H > 512 in bf16) runs kernels that read each
 *      channel's filter by its group index, with the backward in two passes
 *      (same results, slower).
 *   D  multiple of 8 (bf16) or 4 (fp32).
 */
DSC_API dsc_status dsc_headwise_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                            int32_t H, const void *x, const void *w, const int32_t *cu_seqlens,
                            int32_t n_seqs, int32_t residual, void *y);

/*
 * Head-wise backward (chain rule of the forward above, for L = <dy, y>):
 *   dx[m,d]   = rho*dy[m,d] + sum_{k<W, m+k in m's sequence} w[m+k, d/H, k] * dy[m+k,d]
 *   dw[n,j,k] = [n-k in n's sequence] * sum_{d=jH}^{jH+H-1} dy[n,d] * x[n-k,d]
 *
 *   x, dy (B,T,D) in;  w (B,T,D/H,W) in;  dx (B,T,D) out;  dw (B,T,D/H,W) out.
 *   Same shape rules as dsc_headwise_fwd.
 */
DSC_API dsc_status dsc_headwise_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                            int32_t H, const void *x, const void *w, const void *dy,
                            const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                            void *dx, void *dw);

/*
 * Rotary position table for the fused calls below.  The rotation is the one of
 * "RoFormer: Enhanced Transformer with Rotary Position Embedding" (Su et al.),
 * Section 3.4.2: pair i of a head (channels 2i, 2i+1) turns by m * theta_i at
 * position m, theta_i = base^(-2i/head_dim).
 *
 *   table  (max_pos, head_dim/2, 2) fp32, out, 16-byte aligned:
 *          table[m][i][0] = cos(m * theta_i), table[m][i][1] = sin(m * theta_i),
 *          each computed in double precision and rounded once to fp32.
 *   head_dim even, 2..65536; base > 0 (10000 is the usual value).
 * The caller owns the table; it depends only on (max_pos, head_dim, base), so
 * one table serves every call with those values.  max_pos = 0 does nothing.
 */
DSC_API dsc_status dsc_rope_table(void *stream, int64_t max_pos, int32_t head_dim, double base, float *table);

/*
 * Head-wise forward followed by the rotary embedding of the query and key
 * channels.  The pages apply the layer (with its residual) to the Q, K and V
 * projections right before the rotary embedding (Methodology, "placement");
 * this call does both in one pass:
 *   s[n,d] = the head-wise forward above (dsc_headwise_fwd),
 *   y[n,h*hd+2i]   = s[n,h*hd+2i] * c - s[n,h*hd+2i+1] * sn      for h*hd < rot,
 *   y[n,h*hd+2i+1] = s[n,h*hd+2i+1] * c + s[n,h*hd+2i] * sn
 *   y[n,d] = s[n,d] for d >= rot,
 * with (c, sn) = table[pos(n)][i] and pos(n) the index of token n inside its
 * own sequence (0 at each sequence start; packed sequences restart).
 *
 *   rot       channels rotated, from channel 0 (query heads then key heads):
 *             a multiple of head_dim in 0..D; rot = 0 is dsc_headwise_fwd.
 *   head_dim  hd, even; a multiple of 8 (bf16) / 4 (fp32), else
 *             DSC_ERR_UNSUPPORTED.
 *   table     from dsc_rope_table with the same head_dim, in; read when
 *             rot > 0.  max_pos must cover every position: max_pos >= T
 *             without cu_seqlens, max_pos >= B*T with it.
 *   Other arguments and rules as dsc_headwise_fwd.
 */
DSC_API dsc_status dsc_headwise_rope_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                 int32_t H, const void *x, const void *w, const int32_t *cu_seqlens,
                                 int32_t n_seqs, int32_t residual, int64_t rot, int32_t head_dim,
                                 const float *table, int64_t max_pos, void *y);

/*
 * Backward of dsc_headwise_rope_fwd for L = <dy, y>.  The rotation is
 * orthogonal, so the layer's output gradient is dy turned back by the same
 * angles (ds = R^T dy, the transposed rotation); dx and dw are then those of
 * dsc_headwise_bwd with ds in place of dy.  Shapes and rules as
 * dsc_headwise_rope_fwd and dsc_headwise_bwd.
 */
DSC_API dsc_status dsc_headwise_rope_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                 int32_t H, const void *x, const void *w, const void *dy,
                                 const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, int64_t rot,
                                 int32_t head_dim, const float *table, int64_t max_pos, void *dx, void *dw);

/*
 * Head-wise layer whose filters are generated on chip from the hidden state.
 * The pages generate the filter of token t by a learned linear map of the
 * current hidden state (Methodology, "parametrization"); with head-wise tying
 * the map yields one W-tap filter per group of H channels:
 *   w[n, g*W + k] = sum_{j<K} h[n, j] * V[g*W + k, j]        (on chip only)
 *   y[n, d]       = the head-wise forward (dsc_headwise_fwd) with these w.
 * The map runs on the matrix cores (bf16 products, fp32 sums) and its result
 * feeds the convolution in the same kernel; w is never written to memory.
 *
 *   h  (B,T,K) in: the hidden state of each token (the layer's own input x,
 *      or another tensor of any width K, e.g. the block's input);
 *   V  (G*W, K) in: the map's weight, row g*W + k producing tap k of group g
 *      (the layout of a linear layer's weight, out x in), G = D/H;
 *   x  (B,T,D) in;  y (B,T,D) out.
 *   DSC_BF16 only (DSC_ERR_UNSUPPORTED otherwise); K a multiple of 8 and
 *   G*W a multiple of 8 (else DSC_ERR_UNSUPPORTED), K <= 2^20; any H
 *   dividing D.  h may be the same buffer as x.  Other arguments and rules
 *   as dsc_headwise_fwd.
 */
DSC_API dsc_status dsc_headwise_gen_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                        int32_t H, int64_t K, const void *h, const void *V, const void *x,
                                        const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *y);

/*
 * The filter generator alone: w[n, c] = sum_{j<K} h[n, j] * V[c, j] for the
 * N rows of h, i.e. the filters that dsc_headwise_gen_fwd forms on chip,
 * written out (w (N, C) bf16 is the (B,T,G,W) filter tensor of
 * dsc_headwise_fwd when C = G*W).  Same matrix-core product and rounding as
 * the fused layer (bf16 operands, fp32 sums, one rounding to bf16).
 *   h (N, K) in;  V (C, K) in;  w (N, C) out.  DSC_BF16 only; K and C
 *   multiples of 8 (else DSC_ERR_UNSUPPORTED); K <= 2^20, C <= 2^24.
 */
DSC_API dsc_status dsc_generate_filters(void *stream, int dtype, int64_t N, int64_t K, int64_t C, const void *h,
                                        const void *V, void *w);

/*
 * Bytes of device workspace dsc_headwise_gen_bwd needs (0 for invalid
 * sizes): the filter gradient dw (B*T, G*W) in bf16, transposed bf16 copies
 * of V, dw and h (the two products read every operand along its reduced
 * dimension), and, when the sum over tokens of dV is split to fill the
 * device, the fp32 partial sums of each split (added in a fixed order).  It
 * depends on the sizes only.
 */
DSC_API size_t dsc_headwise_gen_bwd_workspace_size(int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                                   int32_t H, int64_t K);

/*
 * Backward of dsc_headwise_gen_fwd for L = <dy, y>:
 *   dx = the head-wise dx (dsc_headwise_bwd) with the generated w,
 *   dw[n, g*W+k] = sum_{d in group g, n-k in n's sequence} dy[n,d] * x[n-k,d],
 *   dh[n, j] = sum_c dw[n, c] * V[c, j],    dV[c, j] = sum_n dw[n, c] * h[n, j].
 * w is generated again on chip (not stored by the forward); dw is rounded to
 * bf16 once, in the workspace, and both products read it from there.
 *   dx (B,T,D) bf16 out;  dh (B,T,K) bf16 out;  dV (G*W, K) fp32 out (zero
 *   for an empty batch).  When h is x, the caller adds dh to dx.
 *   workspace: at least dsc_headwise_gen_bwd_workspace_size() bytes, 16-byte
 *   aligned, contents undefined on entry and exit, overlapping no argument.
 * dx, dh and dV are deterministic (no atomics).  Other rules as
 * dsc_headwise_gen_fwd.
 */
DSC_API dsc_status dsc_headwise_gen_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                        int32_t H, int64_t K, const void *h, const void *V, const void *x,
                                        const void *dy, const int32_t *cu_seqlens, int32_t n_seqs,
                                        int32_t residual, void *dx, void *dh, float *dV, void *workspace,
                                        size_t workspace_bytes);

/*
 * Low-rank forward (fused up-projection; Methodology, "parametrization (1)"
 * and Efficient training implementation, fused low-rank kernel):
 *   w[n,d,k] = sum_{r<R} z[n,r] * U[r, d*W+k]          (on chip only)
 *   y[n,d]   = rho*x[n,d] + sum_{k<W, n-k in n's sequence} w[n,d,k] * x[n-k,d]
 *
 *   x (B,T,D) in;  z (B,T,R) in;  U (R, D*W) in, read as (R, D, W);
 *   y (B,T,D) out.  1 <= R <= 128.  D multiple of 8 (bf16) / 4 (fp32).
 */
DSC_API dsc_status dsc_lowrank_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                           int32_t R, const void *x, const void *z, const void *U,
                           const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *y);

/*
 * Bytes of device workspace dsc_lowrank_bwd needs for these sizes and dtype:
 * an fp32 (B*T, R) accumulator of dz for DSC_BF16, nothing (0) for DSC_FP32,
 * whose dz is accumulated in place.  Also returns 0 for invalid sizes.
 */
DSC_API size_t dsc_lowrank_bwd_workspace_size(int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                      int32_t R);

/*
 * Low-rank backward.  With the per-channel filter gradient
 *   dwc[n,d,k] = [n-k in n's sequence] * dy[n,d] * x[n-k,d]   (on chip only):
 *   dx[m,d]      = rho*dy[m,d] + sum_{k<W, m+k in m's sequence} w[m+k,d,k] * dy[m+k,d]
 *   dz[n,r]      = sum_{d,k} U[r, d*W+k] * dwc[n,d,k]
 *   dU[r, d*W+k] = sum_n z[n,r] * dwc[n,d,k]
 *
 *   x, dy (B,T,D) in;  z (B,T,R) in;  U (R, D*W) in;
 *   dx (B,T,D) dtype out;  dz (B,T,R) dtype out;  dU (R, D*W) fp32 out.
 *   workspace: device memory of at least dsc_lowrank_bwd_workspace_size()
 *   bytes, 16-byte aligned, contents undefined on entry and exit; it must not
 *   overlap any argument.  dz and dU are sums over many partial products
 *   accumulated with fp32 atomics: their last bits may differ run to run
 *   (dsc_lowrank_bwd_deterministic below gives reproducible ones).
 */
DSC_API dsc_status dsc_lowrank_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                           int32_t R, const void *x, const void *z, const void *U, const void *dy,
                           const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *dx,
                           void *dz, float *dU, void *workspace, size_t workspace_bytes);

/*
 * Low-rank forward followed by the rotary embedding of the query and key
 * channels: the fused low-rank layer of the Q, K and V projections right
 * before the rotary embedding (Methodology, "placement"; the rotation of
 * RoFormer, Section 3.4.2) in one pass:
 *   s[n,d] = the low-rank forward above (dsc_lowrank_fwd),
 *   y[n,d] = s[n,d] turned pair by pair at token n's position inside its own
 *            sequence for d < rot, exactly as dsc_headwise_rope_fwd turns it;
 *   y[n,d] = s[n,d] for d >= rot.
 * The rotation acts on the fp32 result before its one rounding to the dtype.
 *   rot, head_dim, table, max_pos  as dsc_headwise_rope_fwd (rot = 0 is
 *   dsc_lowrank_fwd).  Other arguments and rules as dsc_lowrank_fwd.
 */
DSC_API dsc_status dsc_lowrank_rope_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                        int32_t R, const void *x, const void *z, const void *U,
                                        const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, int64_t rot,
                                        int32_t head_dim, const float *table, int64_t max_pos, void *y);

/*
 * Backward of dsc_lowrank_rope_fwd for L = <dy, y>: the layer's output
 * gradient is dy turned back (ds = R^T dy, the transposed rotation), and dx,
 * dz and dU are those of dsc_lowrank_bwd with ds in place of dy.  For DSC_BF16
 * shapes served by the matrix-core backward, ds is formed on chip and rounded
 * to bf16 before it enters the products (like every matrix-core operand);
 * elsewhere it stays fp32.  The workspace that dsc_lowrank_bwd_workspace_size
 * reports suffices.  rot = 0 is dsc_lowrank_bwd.  Other arguments, results
 * and errors as dsc_lowrank_rope_fwd and dsc_lowrank_bwd (dz and dU summed
 * with fp32 atomics).
 */
DSC_API dsc_status dsc_lowrank_rope_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                        int32_t R, const void *x, const void *z, const void *U, const void *dy,
                                        const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, int64_t rot,
                                        int32_t head_dim, const float *table, int64_t max_pos, void *dx,
                                        void *dz, float *dU, void *workspace, size_t workspace_bytes);

/*
 * The low-rank backward above for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): no workspace argument; the fp32 dz accumulator lives
 * in a scratch array built into the library, one per device, held by the
 * process until it ends.  Nothing is allocated by the call.
 *   Limit: B*T*R <= 4,194,304 (16 MiB of fp32); larger sizes return
 *   DSC_ERR_WORKSPACE before any HIP call.  (DSC_FP32 needs no scratch.)
 *   The scratch of the device current at the call is used: the stream must
 *   belong to that device.  Calls that overlap in time on one device race
 *   on its scratch; serialise them (one stream, or events).  The scratch is
 *   cleared by a kernel of the call before use and keeps the last call's
 *   contents afterwards.
 * Other arguments, results and errors as dsc_lowrank_bwd (dz and dU are
 * summed with fp32 atomics).
 */
DSC_API dsc_status dsc_lowrank_bwd_noalloc(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                           int32_t R, const void *x, const void *z, const void *U,
                                           const void *dy, const int32_t *cu_seqlens, int32_t n_seqs,
                                           int32_t residual, void *dx, void *dz, float *dU);

/*
 * Bytes of device workspace dsc_lowrank_bwd_deterministic needs for these
 * sizes and dtype (0 for invalid sizes, and where no workspace is needed).
 * It depends on the sizes and dtype only, not on the device: for DSC_BF16
 * shapes that the matrix-core kernel serves (R <= 32, or R <= 64 with W <= 4)
 * it holds one fp32 (B*T, R) region of dz per block of 128 channels and one
 * fp32 (R, D*W) region of dU per token chunk of the work split; otherwise 0.
 * At B*T = 16384, D = 2304, W = 4, R = 32 that is about 55 MB.
 */
DSC_API size_t dsc_lowrank_bwd_deterministic_workspace_size(int dtype, int64_t B, int64_t T, int64_t D,
                                                            int32_t W, int32_t R);

/*
 * The low-rank backward above with dz and dU summed in one fixed order, so
 * that equal inputs give bitwise equal outputs on every call and on every
 * device.  The same per-block partial sums as dsc_lowrank_bwd are formed;
 * instead of fp32 atomics into one accumulator, each block's partials go to
 * a workspace region of their own (each element written once) and a
 * following launch adds the regions in ascending order (dz: channel blocks,
 * dU: token chunks).  Where the generic kernels serve the shape (DSC_FP32,
 * and the other bf16 shapes) one thread forms each dz and dU element,
 * adding its terms in a fixed order.  dx is the same as dsc_lowrank_bwd's.
 * Arguments, layouts and errors as for dsc_lowrank_bwd, with the workspace
 * sized by dsc_lowrank_bwd_deterministic_workspace_size() (may be NULL when
 * that is 0).  Costs extra HBM traffic: the partial regions (about 54 MB
 * at the sizes above) are cleared, written once and read back.
 */
DSC_API dsc_status dsc_lowrank_bwd_deterministic(void *stream, int dtype, int64_t B, int64_t T, int64_t D,
                                                 int32_t W, int32_t R, const void *x, const void *z,
                                                 const void *U, const void *dy, const int32_t *cu_seqlens,
                                                 int32_t n_seqs, int32_t residual, void *dx, void *dz, float *dU,
                                                 void *workspace, size_t workspace_bytes);

/*
 * Static short convolution: the fixed-filter layer that the dynamic one
 * generalises, with one filter per channel, the same at every position.
 * The authors' thread on digg.com ("Custom Triton GPU kernels maintain
 * wall-clock training efficiency") describes it as a depthwise causal
 * convolution of small width.  The gist.science summaries (Performance) set
 * the dynamic kernels' latency against optimised kernels of this layer
 * (causal_conv1d):
 *   y[n,d] = rho*x[n,d] + sum_{k<W, n-k in n's sequence} c[d,k] * x[n-k,d]
 *
 *   x (B,T,D) dtype, in.   c (D,W) dtype, in: tap k weights lag k, so
 *   c[d,0] multiplies the current token (causal_conv1d's weight with its
 *   taps in reverse order).   y (B,T,D) dtype, out.
 *   D multiple of 8 (bf16) / 4 (fp32).
 */
DSC_API dsc_status dsc_static_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                          const void *x, const void *c, const int32_t *cu_seqlens, int32_t n_seqs,
                          int32_t residual, void *y);

/*
 * Static short convolution, backward for L = <dy, y>:
 *   dx[m,d] = rho*dy[m,d] + sum_{k<W, m+k in m's sequence} c[d,k] * dy[m+k,d]
 *   dc[d,k] = sum over all tokens n of [n-k in n's sequence] dy[n,d] * x[n-k,d]
 *
 *   x, dy (B,T,D) in;  c (D,W) in;  dx (B,T,D) dtype out;  dc (D,W) fp32 out.
 *   dc is a sum over every token accumulated with fp32 atomics: its last
 *   bits may differ run to run (dsc_static_bwd_deterministic below gives
 *   reproducible ones).  An empty batch zero-fills dc.
 */
DSC_API dsc_status dsc_static_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                          const void *x, const void *c, const void *dy, const int32_t *cu_seqlens,
                          int32_t n_seqs, int32_t residual, void *dx, float *dc);

/*
 * Bytes of device workspace dsc_static_bwd_deterministic needs: one fp32
 * (D, W) region of dc per group of token tiles of the backward's work split,
 * which depends on the sizes and dtype only (0 for an empty batch and for
 * invalid sizes).  At B*T = 16384, D = 2304, W = 4 (bf16): 64 regions, 2.4 MB.
 */
DSC_API size_t dsc_static_bwd_deterministic_workspace_size(int dtype, int64_t B, int64_t T, int64_t D,
                                                           int32_t W);

/*
 * The static backward above with dc summed in one fixed order, so that equal
 * inputs give bitwise equal dc on every call and every device.  Each block
 * of the backward adds its dc partial sums (already summed over its tiles in
 * LDS) into a workspace region of its own group of token tiles, each element
 * written once; a following launch adds the regions in ascending order.  dx
 * is the same as dsc_static_bwd's.  Arguments, layouts and errors as for
 * dsc_static_bwd, plus a workspace of at least
 * dsc_static_bwd_deterministic_workspace_size() bytes, 16-byte aligned,
 * contents undefined on entry and exit, overlapping no argument (may be NULL
 * for an empty batch).
 */
DSC_API dsc_status dsc_static_bwd_deterministic(void *stream, int dtype, int64_t B, int64_t T, int64_t D,
                                                int32_t W, const void *x, const void *c, const void *dy,
                                                const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                                                void *dx, float *dc, void *workspace, size_t workspace_bytes);

/*
 * Decoding: one new token per sequence, B sequences, with a rolling state.
 * The authors note that inference needs engineering of its own (gist.science
 * technical summary, Significado y Reivindicaciones).  The step is the
 * forward above evaluated at each sequence's newest token:
 *   y[b,d] = rho*x[b,d] + w(b)_{d,0}*x[b,d] + sum_{k=1}^{W-1} w(b)_{d,k}*state[b,k-1,d]
 * then the state shifts by one token:
 *   state[b,0,d] <- x[b,d],  state[b,i,d] <- state[b,i-1,d] (i >= 1).
 *
 *   state (B, W-1, D) dtype, read and then overwritten in place (the one
 *         in/out argument of the library): state[b,i,d] is the input of token
 *         t-1-i of sequence b, zero before the sequence's first token.  A new
 *         sequence starts from zeros; a prefill hands over its last W-1
 *         inputs with dsc_state_from_prefill.  NULL when W = 1 (no slots).
 *   x, y (B, D) dtype.  D multiple of 8 (bf16) / 4 (fp32).  B may be 0;
 *         B*D < 2^31.
 *   No argument may overlap another (state is not an alias of x or y).
 */

/* Head-wise decoding step: w (B, D/H, W), w(b)_{d,k} = w[b, d/H, k], any H
 * with D % H == 0. */
DSC_API dsc_status dsc_headwise_decode(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t H,
                               const void *x, const void *w, void *state, int32_t residual, void *y);

/*
 * One decoding step of the head-wise layer followed by the rotary embedding of
 * the query and key channels: the serving form of dsc_headwise_rope_fwd.
 * y is dsc_headwise_decode's output turned pair by pair (channels 2i, 2i+1 of
 * each head of head_dim, channels < rot) by positions[b] * theta_i, with the
 * cos / sin of table row positions[b]; the state update is that of
 * dsc_headwise_decode.
 *
 *   positions  (B,) int32, in, device memory: the index of sequence b's new
 *              token inside its sequence (after a prefill of L tokens, the
 *              first step has position L).  A position outside [0, max_pos)
 *              has no table row: that sequence's rotated channels of y are
 *              set to NaN (the table is never read out of bounds).
 *   rot, head_dim, table, max_pos  as dsc_headwise_rope_fwd (rot = 0 is
 *              dsc_headwise_decode; head_dim is still required).
 *   Other arguments and rules as dsc_headwise_decode.
 */
DSC_API dsc_status dsc_headwise_rope_decode(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t H,
                                    const void *x, const void *w, void *state, int32_t residual, int64_t rot,
                                    int32_t head_dim, const float *table, int64_t max_pos,
                                    const int32_t *positions, void *y);

/* Low-rank decoding step: z (B, R), U (R, D*W), w(b)_{d,k} = sum_r z[b,r] U[r, d*W+k]
 * formed on chip.  1 <= R <= 128. */
DSC_API dsc_status dsc_lowrank_decode(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t R,
                              const void *x, const void *z, const void *U, void *state, int32_t residual,
                              void *y);

/* State after a prefill: for every sequence s of the (B,T,D) inputs x (rows,
 * or the cu_seqlens sequences as above), state[s,i,d] = x of the sequence's
 * token end-1-i, or 0 when the sequence has fewer than i+1 tokens.  state is
 * (S, W-1, D) with S = n_seqs (or B without cu_seqlens); nothing is written
 * when W = 1 or B*T = 0. */
DSC_API dsc_status dsc_state_from_prefill(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                  const void *x, const int32_t *cu_seqlens, int32_t n_seqs, void *state);

/* Static name of a status code. */
DSC_API const char *dsc_status_string(int status);

/* Description of the calling thread's most recent failed call ("" if none). */
DSC_API const char *dsc_last_error(void);

/* DSC_ABI_VERSION of the loaded library. */
DSC_API int dsc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSC_H */
