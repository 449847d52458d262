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
    // rotary embedding (ROPE kernels only): channels [0, rot), heads of hd,
    // table (npos, hd/2, 2) of cos, sin
    const float *rope;
    int32_t rot, hd, npos;
};

constexpr int kBlock = 256;

// Cache policy of the low-rank kernels' activation streams: bit 1 x loads,
// 2 y stores (forward), 4 dy loads, 8 dx stores (backward); set bits take
// the nontemporal policy.
#ifndef DSC_LR_NT
#define DSC_LR_NT 13
#endif
constexpr bool kLrNtX = (DSC_LR_NT & 1) != 0;
constexpr bool kLrNtY = (DSC_LR_NT & 2) != 0;
constexpr bool kLrNtG = (DSC_LR_NT & 4) != 0;
constexpr bool kLrNtDx = (DSC_LR_NT & 8) != 0;
constexpr int kMaxTokPerWave = 4096;                          // token walk length cap
constexpr int kSeqWords = (kMaxTokPerWave + 128) / 32 + 2;    // sequence-start bits per wave

// DPP controls (row = 16 lanes): lane i of a row reads lane i-k (shr) or
// lane (i-k) mod 16 (ror).  With lane = token inside a 16-token step, this
// moves the values of token t-K to token t, the first K tokens taking the
// last K of the previous step (prev).
template <int K>
__device__ __forceinline__ uint32_t shift_in_row(uint32_t cur, uint32_t prev) {
    const int rot = __builtin_amdgcn_mov_dpp((int)prev, 0x120 + K, 0xf, 0xf, true);
    return (uint32_t)__builtin_amdgcn_update_dpp(rot, (int)cur, 0x110 + K, 0xf, 0xf, false);
}

// Shift back by a tap k (1 <= k < W, known after unrolling) of four packed
// registers: out = cur moved k tokens later, the first k taken from prev.
template <int W, int K = 1>
__device__ __forceinline__ void shift_back4(int k, const uint32_t (&cur)[4], const uint32_t (&prev)[4],
                                            uint32_t (&out)[4]) {
    if constexpr (K < W) {
        if (k == K) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = shift_in_row<K>(cur[i], prev[i]);
        } else {
            shift_back4<W, K + 1>(k, cur, prev, out);
        }
    }
}

// Shift ahead by K tokens: token t takes the value of token t+K, the last K
// of the row taken from the next step (next).
template <int K>
__device__ __forceinline__ uint32_t shift_ahead_in_row(uint32_t cur, uint32_t next) {
    const int rot = __builtin_amdgcn_mov_dpp((int)next, 0x120 + (16 - K), 0xf, 0xf, true);
    return (uint32_t)__builtin_amdgcn_update_dpp(rot, (int)cur, 0x100 + K, 0xf, 0xf, false);
}

// Shift by a tap k (1 <= k < W, known after unrolling) of four packed registers.
template <int W, int K = 1>
__device__ __forceinline__ void shift_ahead4(int k, const uint32_t (&cur)[4], const uint32_t (&next)[4],
                                             uint32_t (&out)[4]) {
    if constexpr (K < W) {
        if (k == K) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = shift_ahead_in_row<K>(cur[i], next[i]);
        } else {
            shift_ahead4<W, K + 1>(k, cur, next, out);
        }
    }
}

// The same shifts of two packed registers.
template <int W, int K = 1>
__device__ __forceinline__ void shift_back2(int k, const uint32_t (&cur)[2], const uint32_t (&prev)[2],
                                            uint32_t (&out)[2]) {
    if constexpr (K < W) {
        if (k == K) {
            out[0] = shift_in_row<K>(cur[0], prev[0]);
            out[1] = shift_in_row<K>(cur[1], prev[1]);
        } else {
            shift_back2<W, K + 1>(k, cur, prev, out);
        }
    }
}

template <int W, int K = 1>
__device__ __forceinline__ void shift_ahead2(int k, const uint32_t (&cur)[2], const uint32_t (&next)[2],
                                             uint32_t (&out)[2]) {
    if constexpr (K < W) {
        if (k == K) {
            out[0] = shift_ahead_in_row<K>(cur[0], next[0]);
            out[1] = shift_ahead_in_row<K>(cur[1], next[1]);
        } else {
            shift_ahead2<W, K + 1>(k, cur, next, out);
        }
    }
}

__device__ __forceinline__ bf16x8 bf16x8_from_u32(const uint32_t (&v)[4]) {
    uint4 q = make_uint4(v[0], v[1], v[2], v[3]);
    return __builtin_bit_cast(bf16x8, q);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane i receives element (i & 3) of the 8-byte chunks addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4.  Addressing lane i at row base + i/4,
// column col0 + 4*(i & 3) of a row-major [row][col] bf16 array therefore
// returns rows base .. base+3 of column col0 + i.
__device__ __forceinline__ uint2 lds_read_tr(const unsigned char *addr) {
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(addr));
    return __builtin_bit_cast(uint2, v);
}

// Compile-time switch of a step body between its masked and unmasked copies.
template <bool V> struct MaskTag { static constexpr bool value = V; };

// Position of a lane's token inside its sequence, for a walk in 16-token
// steps taken in order.  `start` is the first token of the sequence in
// effect before the step (wave-uniform); the step's own starts come from the
// walk's bitmap.  pos_and_advance returns the lane's position at step
// token nstep + tok and moves `start` past the step.
struct SeqPos {
    int64_t start;
    template <int kWords>
    __device__ __forceinline__ int64_t pos_and_advance(const StartBits<kWords> &bits, int64_t nstep, int tok) {
        const uint32_t w16 = __builtin_amdgcn_readfirstlane(bits.window(nstep)) & 0xffffu;
        const uint32_t m = w16 & ((2u << tok) - 1u);  // starts among tokens nstep .. nstep + tok
        const int64_t s = m ? nstep + (31 - __builtin_clz(m)) : start;
        if (w16) start = nstep + (31 - __builtin_clz(w16));
        return nstep + tok - s;
    }
};

// cos, sin of the VEC/2 pairs of VEC channels starting at channel ch (a
// multiple of VEC, so all in one head) of a token at position pos.  Any
// channel reads the entry of its place in its head, so callers may load for
// channels past rot and skip the turn; pos is clamped into the table
// (positions past it belong to tokens past the walk, whose values are never
// stored).
template <int VEC>
__device__ __forceinline__ void rope_cs(const LrParams &p, int64_t pos, int64_t ch, float (&cs)[VEC]) {
    const int64_t m = pos < 0 ? 0 : (pos >= p.npos ? p.npos - 1 : pos);
    load_turn<VEC>(p.rope + m * p.hd + (int32_t)(ch % p.hd), cs);
}

// cos, sin of a lane's 4 pairs (8 channels from ch) at its token's position,
// carried along a walk of 16-token steps: a token 16 or more positions into
// its sequence turns the value its lane held one step earlier (the token 16
// before, same sequence) by 16 positions, angle addition with table row 16.
// Tokens within 16 of their sequence start, and the walk's first step, read
// the table; steps with none of those (the test is wave-uniform) issue no
// memory load, so the streams' prefetch depth stays intact.  Each turn adds
// about one fp32 rounding: over a 4096-token walk well under bf16 resolution.
struct RopeCarry {
    float c[8];
    __device__ __forceinline__ void start(const LrParams &p, int64_t pos, int64_t ch) { rope_cs<8>(p, pos, ch, c); }
    // r16: cos, sin of 16 positions for the lane's 4 pairs (table row 16);
    // restart: some token of the step is within 16 of its sequence start (a
    // wave-uniform flag from the start bitmap).  In such a step every lane
    // loads (position clamped) and a select consumes the load inside the
    // branch, so the wait for it stays there: a load whose value lived on past
    // the branch would make every step wait for it, and with it for the
    // streams' prefetched loads.
    __device__ __forceinline__ void advance(const LrParams &p, int64_t pos, int64_t ch, const float (&r16)[8],
                                            bool restart) {
        compose<8>(c, r16);
        if (restart) {
            float t[8];
            rope_cs<8>(p, pos < 16 ? pos : 0, ch, t);
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = pos < 16 ? t[e] : c[e];
        }
    }
};

// Whether a step of 16 tokens from nstep has a token within 16 positions of
// its sequence start: a start among tokens nstep - 15 .. nstep + 15.
template <int kWords>
__device__ __forceinline__ bool rope_restart(const StartBits<kWords> &bits, int64_t nstep) {
    return (__builtin_amdgcn_readfirstlane(bits.window(nstep - 15)) & 0x7fffffffu) != 0u;
}

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
                // every lane loads (from U's start when out of range) and zeroes by a
                // mask: a branch per element would wait for each load in turn
                const bool ok = r < R && ch < D;
                const uint16_t m = (uint16_t)keep_mask(ok);
                load_taps<W>(U + (ok ? ((int64_t)r * D + ch) * W : 0), v);
#pragma unroll
                for (int k = 0; k < W; ++k) ua[k][t][c][e] = __builtin_bit_cast(__bf16, (uint16_t)(v[k] & m));
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
    p.rope = pr.rope;
    p.rot = (int32_t)pr.rot;
    p.hd = pr.hd;
    p.npos = (int32_t)pr.max_pos;
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

// The reproducible backward splits the work as the fast one would on a
// 256-CU device with one block per CU, on every device, so that its order
// of summation is the same everywhere.
constexpr int64_t kDetSlots = 256;

constexpr int64_t kWaveFixedTokens = 64;  // a forward wave's set-up, in tokens of walk

}  // namespace
}  // namespace dsc
