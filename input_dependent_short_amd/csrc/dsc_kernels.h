// dsc_kernels.h -- launchers of the dynamic short convolution kernels.
// Internal to libdsc.so; the public surface is include/dsc.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsc_common.h"

namespace dsc {

enum class Dtype { F32 = 0, BF16 = 1 };

// Head-wise problem (validated by the API layer).
struct HwProblem {
    Dtype dtype;
    int64_t N, T, D;
    int32_t W, H;
    const void *x, *w, *dy;
    void *y, *dx, *dw;
    const int32_t *cu;
    int32_t n_seqs;
    int32_t residual;
    // Rotary embedding after the layer (headwise_rope_* only): channels
    // [0, rot) in heads of hd, cos / sin table (max_pos, hd/2, 2).
    int64_t rot;
    int32_t hd;
    const float *rope;
    int64_t max_pos;  // table rows
};

// Low-rank problem.
struct LrProblem {
    Dtype dtype;
    int64_t N, T, D;
    int32_t W, R;
    const void *x, *z, *U, *dy;
    void *y, *dx, *dz;
    float *dU;
    float *dz_acc;  // fp32 accumulator (workspace) when dz is not fp32
    const int32_t *cu;
    int32_t n_seqs;
    int32_t residual;
    // Rotary embedding after the layer (lowrank_rope_* only): channels
    // [0, rot) in heads of hd, cos / sin table (max_pos, hd/2, 2).
    int64_t rot = 0;
    int32_t hd = 0;
    const float *rope = nullptr;
    int64_t max_pos = 0;
};

// Head-wise layer whose filters are generated on chip from the hidden state
// (generator.hip): w[n, g*W + k] = sum_j h[n, j] V[g*W + k, j], bf16 only.
struct GenProblem {
    int64_t N, T, D;
    int32_t W, H;
    int64_t K;  // hidden width
    const void *h, *V, *x, *dy;
    void *y, *dx, *dh;
    float *dV;
    void *dw;  // backward workspace (headwise_gen_bwd_workspace bytes), the filter gradient first
    const int32_t *cu;
    int32_t n_seqs;
    int32_t residual;
};
hipError_t headwise_gen_fwd(const GenProblem &p, hipStream_t s);
// Workspace bytes of headwise_gen_bwd (p.dw points at it): the filter
// gradient, the transposed operands of dh and dV, and dV's split partials.
size_t headwise_gen_bwd_workspace(int64_t N, int64_t D, int32_t W, int32_t H, int64_t K);
hipError_t headwise_gen_bwd(const GenProblem &p, hipStream_t s);
// w (N x C) = h (N x K) . V (C x K)^T in bf16 (fp32 sums), on the same
// matrix-core GEMM as the fused layer.
hipError_t generate_filters(const uint16_t *h, const uint16_t *V, int64_t N, int64_t K, int64_t C, uint16_t *w,
                            hipStream_t s);

// Static short convolution: one filter per channel, the same at every token.
struct StProblem {
    Dtype dtype;
    int64_t N, T, D;
    int32_t W;
    const void *x, *c, *dy;
    void *y, *dx;
    float *dc;
    const int32_t *cu;
    int32_t n_seqs;
    int32_t residual;
};

// One decoding step (one token per sequence) with a rolling state.
struct DecProblem {
    Dtype dtype;
    int64_t B, D;
    int32_t W, H, R;
    bool lowrank;
    const void *x, *w, *z, *U;
    void *state, *y;
    int32_t residual;
    // head-wise only: rotary embedding of y's channels [0, rot) at positions
    // pos (B,), from the table (max_pos, hd/2, 2); rot = 0 for none
    int64_t rot;
    int32_t hd;
    const float *rope;
    int64_t max_pos;
    const int32_t *pos;
};

// Head-wise: whether the kernels of headwise_impl.h serve (dtype, H); every
// other H with D % H == 0 runs the kernels of headwise_any.hip.
bool headwise_fast(Dtype dt, int32_t H);
// The layer (rope false) or the layer with the rotary embedding for any H.
hipError_t headwise_any(const HwProblem &p, hipStream_t s, bool bwd, bool rope);

hipError_t headwise_fwd(const HwProblem &p, hipStream_t s);
hipError_t headwise_bwd(const HwProblem &p, hipStream_t s);
// The same layer followed by the rotary embedding of channels [0, p.rot).
hipError_t headwise_rope_fwd(const HwProblem &p, hipStream_t s);
hipError_t headwise_rope_bwd(const HwProblem &p, hipStream_t s);
// table[(m*hd/2 + i)*2 + {0,1}] = {cos, sin}(m * base^(-2i/hd)), m < max_pos.
hipError_t rope_table(int64_t max_pos, int32_t hd, double base, float *table, hipStream_t s);

// split_ok false keeps dz inside the matrix-core backward (workspace: one
// fp32 (N, R) accumulator), as the allocation-free entry point needs.
size_t lowrank_bwd_workspace(Dtype dt, int64_t N, int64_t D, int32_t W, int32_t R, bool split_ok = true);

// dz of the low-rank backward as its own launches (lowrank_dz.hip): a
// tap-major copy of U (ut_elems bf16) and fp32 partial sums, one (N, R)
// region per split of the channels (S of them, cper channels each), added in
// ascending order afterwards.  The split depends on the sizes only.
struct LrDzPlan {
    int64_t ntb, cper;
    int32_t S;
    int64_t ut_elems, part_floats;
};
LrDzPlan lowrank_dz_plan(int64_t N, int64_t D, int32_t W, int32_t R);
bool lowrank_dz_supported(int32_t W, int32_t R);
hipError_t lowrank_dz_partials(const LrProblem &pr, const LrDzPlan &pl, uint16_t *Ut, float *parts, hipStream_t st);
hipError_t lowrank_fwd(const LrProblem &p, hipStream_t s);
// Wide bf16 forward (R <= 64); sets *used to false when the shape is left to
// the other kernels, which then run instead.
hipError_t lowrank_fwd_wide(const LrProblem &p, hipStream_t s, bool *used);
hipError_t lowrank_bwd(const LrProblem &p, hipStream_t s, bool split_ok = true);
// The low-rank layer followed by the rotary embedding of channels [0, p.rot)
// (the backward turns dy back first); the backward's workspace is that of
// lowrank_bwd_workspace(..., split_ok = false).
hipError_t lowrank_rope_fwd(const LrProblem &p, hipStream_t s);
hipError_t lowrank_rope_bwd(const LrProblem &p, hipStream_t s);
// Reproducible backward: dz and dU summed in one fixed order (dz_acc = its
// workspace of lowrank_bwd_det_workspace bytes, may be null when that is 0).
size_t lowrank_bwd_det_workspace(Dtype dt, int64_t N, int64_t D, int32_t W, int32_t R);
hipError_t lowrank_bwd_det(const LrProblem &p, hipStream_t s);
hipError_t static_fwd(const StProblem &p, hipStream_t s);
// Zero-fills dc, then runs the backward (dx and the fp32 sums of dc); with
// N = 0 only the zero-fill runs.
hipError_t static_bwd(const StProblem &p, hipStream_t s);
// Fixed-order backward: dc of each token-tile group in a region of ws (bytes
// from static_bwd_det_workspace), the regions then added in order into dc.
size_t static_bwd_det_workspace(Dtype dt, int64_t N, int64_t D, int32_t W);
hipError_t static_bwd_det(const StProblem &p, float *ws, hipStream_t s);

hipError_t decode_step(const DecProblem &p, hipStream_t s);
// Last W-1 inputs of every sequence of a prefill into the state (S, W-1, D).
hipError_t state_from_prefill(Dtype dt, const void *x, const int32_t *cu, int32_t n_seqs, int64_t B, int64_t T,
                              int64_t D, int32_t W, void *state, hipStream_t s);

// Allocation-free low-rank backward: the device address of this device's
// file-scope scratch (kNoallocScratchFloats fp32 values), taken once per
// device (noalloc.hip).
constexpr int64_t kNoallocScratchFloats = (int64_t)4 << 20;  // 16 MiB: B*T*R <= 4,194,304
hipError_t noalloc_scratch(float **out);

// Streaming measurement kernel (stream.hip): reads read_bytes and writes
// write_bytes in 16-byte units; blocks <= 0 takes one round of resident
// workgroups.
hipError_t stream_probe(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes, int unroll, bool lnt,
                        bool snt, bool chunked, int64_t blocks, hipStream_t s);

// Zero-fills n fp32 values (16-byte aligned); the backward of an empty batch.
hipError_t lowrank_zero(float *p, int64_t n, hipStream_t s);
// Zeroes two fp32 arrays in one launch; rounds n fp32 values to bf16.
hipError_t lowrank_zero2(float *a, int64_t na, float *b, int64_t nb, hipStream_t s);
hipError_t lowrank_round_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t s);
// Backward of the bf16 low-rank layer for 32 < R <= 64 and 2 <= W <= 4 with
// each 32-channel slice split between two waves by channels
// (lowrank_taps.hip); workspace as lowrank_bwd's (an fp32 (N, R) dz
// accumulator).  det: the reproducible split (dz per channel group and dU per
// token chunk in regions of dz_acc, lowrank_bwd_taps_det_workspace bytes,
// added in order).  _rope: the layer followed by the rotary embedding (p.rope,
// p.rot, p.hd, p.npos set), fast split only.
bool lowrank_bwd_taps_supported(Dtype dt, int64_t D, int32_t W, int32_t R);
hipError_t lowrank_bwd_taps(const LrProblem &p, hipStream_t s, bool det);
hipError_t lowrank_bwd_taps_rope(const LrProblem &p, hipStream_t s);
size_t lowrank_bwd_taps_det_workspace(int64_t N, int64_t D, int32_t W, int32_t R);
// dst = sum over parts j (ascending) of src[j*stride + i], as fp32 or rounded to bf16
hipError_t lowrank_sum_parts(const float *src, int64_t nparts, int64_t stride, float *dst_f32, uint16_t *dst_bf16,
                             int64_t n, hipStream_t s);

}  // namespace dsc
