// rope.hip -- the head-wise layer followed by the rotary position embedding
// of the query and key channels, and the cos / sin table it reads.
//
// The pages put the layer, with its residual, on the query, key and value
// projections right before the rotary embedding ("Dynamic Short Convolutions
// Improve Transformers", gist.science technical summary, Methodology:
// placement).  The rotation is that of "RoFormer: Enhanced Transformer with
// Rotary Position Embedding" (Su et al., Section 3.4.2): pair i = channels
// (2i, 2i+1) of a head of hd channels turns by m * theta_i at position m,
// theta_i = base^(-2i/hd).  Fusing it into the layer saves a read and a write
// of the rotated channels in both directions; the kernels are those of
// headwise_impl.h with the rotation switched on.
#include "headwise_impl.h"

namespace dsc {
namespace {

// One thread per (position, pair).  The angle and its cos / sin are taken in
// double precision and rounded once to fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *table, int64_t entries, int32_t half, double base) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= entries) return;
    const int64_t m = idx / half;
    const int32_t i = (int32_t)(idx - m * half);
    const double ang = (double)m * pow(base, -2.0 * i / (2 * half));
    double sv, cv;
    sincos(ang, &sv, &cv);
    table[idx] = make_float2((float)cv, (float)sv);
}

}  // namespace

hipError_t headwise_rope_fwd(const HwProblem &p, hipStream_t s) {
    if (!headwise_fast(p.dtype, p.H)) return headwise_any(p, s, false, true);
    return p.dtype == Dtype::BF16 ? dispatch<BF16, true>(p, s, false) : dispatch<F32, true>(p, s, false);
}

hipError_t headwise_rope_bwd(const HwProblem &p, hipStream_t s) {
    if (!headwise_fast(p.dtype, p.H)) return headwise_any(p, s, true, true);
    return p.dtype == Dtype::BF16 ? dispatch<BF16, true>(p, s, true) : dispatch<F32, true>(p, s, true);
}

hipError_t rope_table(int64_t max_pos, int32_t hd, double base, float *table, hipStream_t s) {
    const int64_t entries = max_pos * (hd / 2);
    const int64_t blocks = (entries + 255) / 256;
    if (blocks)
        hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<float2 *>(table), entries, hd / 2, base);
    return hipGetLastError();
}

}  // namespace dsc
