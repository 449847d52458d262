// lowrank_common.h -- pieces shared by the low-rank kernels of lowrank.hip
// and lowrank_fwd.hip: kernel parameters, U operand loaders and the
// launch-size helpers.  Internal to libdsc.so.
#pragma once

#include <atomic>

#include "dsc_kernels.h"

namespace dsc {
namespace {

struct LrParams {
    const void *x, *z, *U, *dy;
    void *y, *dx, *dz;
    float *dU, *dzacc;
    SeqMap seq;
    int64_t N, D;
    int32_t R;
    float rho;
    uint32_t rmask;  // all ones with the residual term, else zero
    int64_t nchunks;
    // Backward partial sums: the matrix-core backward adds its dz of channel
    // group g at dzacc + g*dz_gstride and its dU of token chunk c at
    // dU + c*du_cstride.  Both are 0 when the partials share one accumulator.
    int64_t dz_gstride, du_cstride;
};

constexpr int kBlock = 256;
constexpr int kMaxTokPerWave = 4096;                          // token walk length cap
constexpr int kSeqWords = (kMaxTokPerWave + 128) / 32 + 2;    // sequence-start bits per wave

// ---------------------------------------------------------------- U operands

// W consecutive bf16 values of U (the taps of one rank and channel) as raw
// bits, with the widest accesses that the alignment allows: the offset
// (r*D + ch)*W*2 is a multiple of the largest power of two dividing 2W
// because D % 8 == 0.
template <int W>
__device__ __forceinline__ void load_taps(const uint16_t *p, uint16_t (&v)[W]) {
    constexpr int PER = pow2_align(2 * W) / 2;  // elements per access
#pragma unroll
    for (int i = 0; i < W; i += PER) {
        if constexpr (PER == 8) {
            const uint4 q = *reinterpret_cast<const uint4 *>(p + i);
            const uint32_t h[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[i + 2 * j] = (uint16_t)(h[j] & 0xffffu);
                v[i + 2 * j + 1] = (uint16_t)(h[j] >> 16);
            }
        } else if constexpr (PER == 4) {
            const uint2 q = *reinterpret_cast<const uint2 *>(p + i);
            v[i] = (uint16_t)(q.x & 0xffffu); v[i + 1] = (uint16_t)(q.x >> 16);
            v[i + 2] = (uint16_t)(q.y & 0xffffu); v[i + 3] = (uint16_t)(q.y >> 16);
        } else if constexpr (PER == 2) {
            const uint32_t q = *reinterpret_cast<const uint32_t *>(p + i);
            v[i] = (uint16_t)(q & 0xffffu); v[i + 1] = (uint16_t)(q >> 16);
        } else {
            v[i] = p[i];
        }
    }
}

// A operand of w = z U for every tap k, kept in registers: rows are the
// channels of a 32-channel slice (tile t, row i <-> channel
// d0 + 8(i>>2) + 4t + (i&3)), K is rank 32c + 8(lane>>4) + e.  Zero outside R
// and D.
template <int W, int RC>
__device__ __forceinline__ void load_u_rows(const uint16_t *U, int R, int64_t D, int64_t d0, int lane,
                                            bf16x8 (&ua)[W][2][RC]) {
    const int i16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t ch = d0 + 8 * (i16 >> 2) + 4 * t + (i16 & 3);
#pragma unroll
        for (int c = 0; c < RC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 32 * c + 8 * q + e;
                uint16_t v[W];
#pragma unroll
                for (int k = 0; k < W; ++k) v[k] = 0;
                if (r < R && ch < D) load_taps<W>(U + ((int64_t)r * D + ch) * W, v);
#pragma unroll
                for (int k = 0; k < W; ++k) ua[k][t][c][e] = __builtin_bit_cast(__bf16, v[k]);
            }
    }
}

template <class E>
LrParams make_params(const LrProblem &pr) {
    LrParams p;
    p.x = pr.x; p.z = pr.z; p.U = pr.U; p.dy = pr.dy;
    p.y = pr.y; p.dx = pr.dx; p.dz = pr.dz;
    p.dU = pr.dU; p.dzacc = pr.dz_acc;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N; p.D = pr.D; p.R = pr.R;
    p.rho = pr.residual ? 1.f : 0.f;
    p.rmask = pr.residual ? 0xffffffffu : 0u;
    p.nchunks = pr.D / E::kVec;
    p.dz_gstride = 0;
    p.du_cstride = 0;
    return p;
}

int64_t nblocks(int64_t n) { return (n + kBlock - 1) / kBlock; }

// Walk length of one work item (a wave of the forward, a block of the
// backward): whole groups of `unit` tokens, at most `cap`.  ceil(N / len) *
// `lanes` items run in rounds of `slots` resident items, so the length that
// minimises rounds x (len + fixed cost) is taken (the longest on ties).
int64_t walk_length(int64_t N, int64_t lanes, int64_t slots, int64_t cap, int64_t unit, int64_t fixed) {
    int64_t best = unit, best_cost = -1;
    for (int64_t len = (cap / unit) * unit; len >= unit; len -= unit) {
        const int64_t items = ((N + len - 1) / len) * lanes;
        const int64_t rounds = (items + slots - 1) / slots;
        const int64_t cost = rounds * (len + fixed);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = len;
        }
    }
    return best;
}

// Walk length cap: the LDS sequence bitmap, and stream offsets below 2^30
// (the walk plus the prefetch overrun, in 2-byte elements of D channels).
int64_t walk_cap(int64_t D, int64_t unit, int64_t overrun) {
    const int64_t span = kStreamSpan / (2 * D) - overrun;
    return ((span < kMaxTokPerWave ? span : kMaxTokPerWave) / unit) * unit;
}

constexpr int64_t kWaveFixedTokens = 64;  // a forward wave's set-up, in tokens of walk

}  // namespace
}  // namespace dsc
