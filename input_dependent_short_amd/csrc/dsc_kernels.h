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
};

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

// Head-wise: whether this build has a kernel for (dtype, H).
bool headwise_supported(Dtype dt, int64_t D, int32_t H);

hipError_t headwise_fwd(const HwProblem &p, hipStream_t s);
hipError_t headwise_bwd(const HwProblem &p, hipStream_t s);
// The same layer followed by the rotary embedding of channels [0, p.rot).
hipError_t headwise_rope_fwd(const HwProblem &p, hipStream_t s);
hipError_t headwise_rope_bwd(const HwProblem &p, hipStream_t s);
// table[(m*hd/2 + i)*2 + {0,1}] = {cos, sin}(m * base^(-2i/hd)), m < max_pos.
hipError_t rope_table(int64_t max_pos, int32_t hd, double base, float *table, hipStream_t s);

size_t lowrank_bwd_workspace(Dtype dt, int64_t N, int64_t D, int32_t W, int32_t R);
hipError_t lowrank_fwd(const LrProblem &p, hipStream_t s);
// Wide bf16 forward (R <= 64); sets *used to false when the shape is left to
// the other kernels, which then run instead.
hipError_t lowrank_fwd_wide(const LrProblem &p, hipStream_t s, bool *used);
hipError_t lowrank_bwd(const LrProblem &p, hipStream_t s);
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

// Zero-fills n fp32 values (16-byte aligned); the backward of an empty batch.
hipError_t lowrank_zero(float *p, int64_t n, hipStream_t s);

}  // namespace dsc
