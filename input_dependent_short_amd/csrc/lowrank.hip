// lowrank.hip -- low-rank dynamic short convolution for gfx950: the filter of
// token n is generated on chip from its rank-R coefficients and never stored.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: parametrization (1) low-rank factorisation;
// Efficient training implementation: the fused low-rank kernel reads z and U,
// forms zU on chip and convolves at once):
//   w[n,d,k] = sum_{r<R} z[n,r] * U[r, d*W+k]
//   y[n,d]   = rho*x[n,d] + sum_{k<W, n-k in seq(n)} w[n,d,k] * x[n-k,d]
// Backward for L = <dy, y>, with dwc[n,d,k] = [n-k in seq(n)] dy[n,d] x[n-k,d]:
//   dx[m,d]      = rho*dy[m,d] + sum_{k<W, m+k in seq(m)} w[m+k,d,k] dy[m+k,d]
//   dz[n,r]      = sum_{d,k} U[r,d*W+k] dwc[n,d,k]
//   dU[r,d*W+k]  = sum_n z[n,r] dwc[n,d,k]
//
// This file holds the backward kernels, the 32-channel forward kernel and the
// dispatch.  The bf16 forward for R <= 64 runs the wide kernel of
// lowrank_fwd.hip (64 channels per wave, whole-line loads and stores); the
// 32-channel forward below serves R > 64 and very wide D.
//
// 32-channel bf16 forward: the R-wide contraction runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16), one product per tap, C_k = U_k^T (channels x R)
// times Z^T (R x 16 tokens).  Every tap lands in the same accumulator layout
// (lane = token, four channel rows per tile), so the convolution is lane-local:
// y += C_k * x shifted by k tokens, the shift done with DPP row moves inside
// each 16-lane row plus the previous step's registers.  Channel rows are
// permuted so a lane's 8 channels are contiguous: x and y move as 16-byte
// vectors.  U stays in registers for a wave's whole token walk.
//
// The generic kernels (any dtype; fp32 always uses them) evaluate the same
// sums on the vector ALU; dz and dU are reduced with fp32 atomics.
#include "lowrank_common.h"

namespace dsc {
namespace {

// ---------------------------------------------------------------- generic

// One thread per (token, 16-byte channel chunk).  ROPE: channels below p.rot
// of the result are then turned at the token's position in its sequence.
template <class E, int W, bool ROPE = false>
__global__ __launch_bounds__(kBlock) void lr_fwd_generic(LrParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    const int64_t item = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (item >= p.N * p.nchunks) return;
    const int64_t n = item / p.nchunks;
    const int64_t d0 = (item - n * p.nchunks) * VEC;
    const S *x = static_cast<const S *>(p.x);
    const S *z = static_cast<const S *>(p.z);
    const S *U = static_cast<const S *>(p.U);
    const int64_t DW = p.D * W;
    int64_t s, e;
    p.seq.find(n, s, e);

    float xv[VEC], acc[VEC], wv[VEC * W];
    Vec16<E>::load(x + n * p.D + d0, xv);
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = p.rho * xv[c];
#pragma unroll
    for (int i = 0; i < VEC * W; ++i) wv[i] = 0.f;
    for (int r = 0; r < p.R; ++r) {
        const float zr = load_elem<E>(z + n * p.R + r);
        float u[VEC * W];
        Span<E, VEC * W>::template load<pow2_align(W * (int)sizeof(S))>(U + r * DW + d0 * W, u);
#pragma unroll
        for (int i = 0; i < VEC * W; ++i) wv[i] = __builtin_fmaf(zr, u[i], wv[i]);
    }
#pragma unroll
    for (int k = 0; k < W; ++k) {
        if (n - k >= s) {
            float xk[VEC];
            Vec16<E>::load(x + (n - k) * p.D + d0, xk);
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = __builtin_fmaf(wv[c * W + k], xk[c], acc[c]);
        }
    }
    if constexpr (ROPE) {
        if (d0 < p.rot) {
            float cs[VEC];
            rope_cs<VEC>(p, n - s, d0, cs);
            turn<VEC, false>(acc, cs);
        }
    }
    Vec16<E>::store(static_cast<S *>(p.y) + n * p.D + d0, acc);
}

// SUMS: also add this item's dz and dU terms with atomics (else dx only).
// ROPE: dy's channels below p.rot are turned back first (each token at its
// own position), in fp32.
template <class E, int W, bool SUMS = true, bool ROPE = false>
__global__ __launch_bounds__(kBlock) void lr_bwd_generic(LrParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int UALIGN = pow2_align(W * (int)sizeof(S));
    const int64_t item = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (item >= p.N * p.nchunks) return;
    const int64_t m = item / p.nchunks;
    const int64_t d0 = (item - m * p.nchunks) * VEC;
    const S *x = static_cast<const S *>(p.x);
    const S *g = static_cast<const S *>(p.dy);
    const S *z = static_cast<const S *>(p.z);
    const S *U = static_cast<const S *>(p.U);
    const int64_t DW = p.D * W;
    int64_t s, e;
    p.seq.find(m, s, e);
    auto turn_back = [&](float (&v)[VEC], int64_t t) {
        if constexpr (ROPE) {
            if (d0 < p.rot) {
                float cs[VEC];
                rope_cs<VEC>(p, t - s, d0, cs);
                turn<VEC, true>(v, cs);
            }
        }
    };

    // dx: filters of the W tokens m..m+W-1 that read x[m]
    float gm[VEC], acc[VEC];
    Vec16<E>::load(g + m * p.D + d0, gm);
    turn_back(gm, m);
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = p.rho * gm[c];
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const int64_t t = m + k;
        if (t < e) {
            float wk[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) wk[c] = 0.f;
            for (int r = 0; r < p.R; ++r) {
                const float zr = load_elem<E>(z + t * p.R + r);
                float u[VEC * W];
                Span<E, VEC * W>::template load<UALIGN>(U + r * DW + d0 * W, u);
#pragma unroll
                for (int c = 0; c < VEC; ++c) wk[c] = __builtin_fmaf(zr, u[c * W + k], wk[c]);
            }
            float gt[VEC];
            Vec16<E>::load(g + t * p.D + d0, gt);
            turn_back(gt, t);
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = __builtin_fmaf(wk[c], gt[c], acc[c]);
        }
    }
    Vec16<E>::store(static_cast<S *>(p.dx) + m * p.D + d0, acc);
    if constexpr (!SUMS) return;

    // per-channel filter gradient of token m
    float dwc[VEC * W];
#pragma unroll
    for (int k = 0; k < W; ++k) {
        float xk[VEC];
        if (m - k >= s) {
            Vec16<E>::load(x + (m - k) * p.D + d0, xk);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) xk[c] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) dwc[c * W + k] = gm[c] * xk[c];
    }
    for (int r = 0; r < p.R; ++r) {
        float u[VEC * W];
        Span<E, VEC * W>::template load<UALIGN>(U + r * DW + d0 * W, u);
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < VEC * W; ++i) v = __builtin_fmaf(u[i], dwc[i], v);
        atomicAdd(p.dzacc + m * p.R + r, v);
        const float zr = load_elem<E>(z + m * p.R + r);
#pragma unroll
        for (int i = 0; i < VEC * W; ++i) atomicAdd(p.dU + r * DW + d0 * W + i, zr * dwc[i]);
    }
}

// ------------------------------------------------------------- bf16 MFMA

// A operand of dz^T = U_k dwc_k for every tap k: rows are ranks
// 16rt + (lane&15), K is channel d0 + 8(lane>>4) + e.  A lane's 8 channels
// and W taps are 8W consecutive values of U, 16-byte aligned.
template <int W, int RT>
__device__ __forceinline__ void load_u_cols(const uint16_t *U, int R, int64_t D, int64_t d0, int lane,
                                            bf16x8 (&ub)[W][RT]) {
    const int i16 = lane & 15, q = lane >> 4;
    const int64_t ch0 = d0 + 8 * q;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = 16 * rt + i16;
        uint32_t h[4 * W];
        // loads from U's start when out of range, zeroed by a mask (no branch per load)
        const bool ok = r < R && ch0 < D;
        const uint32_t m = keep_mask(ok);
        const uint4 *src = reinterpret_cast<const uint4 *>(U + (ok ? ((int64_t)r * D + ch0) * W : 0));
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const uint4 v = src[j];
            h[4 * j] = v.x & m; h[4 * j + 1] = v.y & m;
            h[4 * j + 2] = v.z & m; h[4 * j + 3] = v.w & m;
        }
#pragma unroll
        for (int idx = 0; idx < 8 * W; ++idx) {  // element idx = channel e * W + tap k
            const uint16_t v = (uint16_t)((idx & 1) ? (h[idx >> 1] >> 16) : (h[idx >> 1] & 0xffffu));
            ub[idx % W][rt][idx / W] = __builtin_bit_cast(__bf16, v);
        }
    }
}


template <int W>
struct Shifted {
    uint32_t v[W][4];
};

template <int W, int K>
__device__ __forceinline__ void fill_shift(Shifted<W> &xs, const uint32_t (&cur)[4], const uint32_t (&prev)[4]) {
    if constexpr (K < W) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xs.v[K][i] = shift_in_row<K>(cur[i], prev[i]);
        fill_shift<W, K + 1>(xs, cur, prev);
    }
}

// Wave tile: 16 tokens (one per lane column) x 32 channels (two 16-row MFMA
// tiles).  Lane l: token l & 15, channel group q = l >> 4 owning channels
// d0 + 8q .. d0 + 8q + 7.  MFMA tile t, row i <-> channel d0 + 8(i>>2) + 4t + (i&3).
// x, z and y move through one raw buffer resource each over the wave's
// token range; a lane's offset is its constant place in a step plus the
// step's offset, and tokens past the range fall outside the resource (loads
// read zero, stores are dropped).  Loads run PF steps ahead in a register
// ring.
template <int W, int RC, int PF, bool RVEC>
__global__ __launch_bounds__(kBlock) void lr_fwd_mfma(LrParams p, int64_t nslices, int64_t tok_per_wave) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kBlock / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tchunk = wave / nslices;
    const int64_t slice = wave - tchunk * nslices;
    const int64_t d0 = slice * 32;
    const int64_t nbeg = tchunk * tok_per_wave;
    if (nbeg >= p.N) return;  // wave-uniform
    const int64_t nend = min(nbeg + tok_per_wave, p.N);
    const int nsteps = (int)((nend - nbeg + 15) / 16);

    const int tok = lane & 15;
    const int q = lane >> 4;
    const int64_t cbase = d0 + 8 * q;
    const bool chan_ok = cbase < p.D;  // D % 8 == 0: a lane's 8 channels are all in or out
    const int R = p.R;
    const int64_t D = p.D;
    const int64_t DW = D * W;

    const uint16_t *U = static_cast<const uint16_t *>(p.U);
    const uint16_t *xg = static_cast<const uint16_t *>(p.x);
    const uint16_t *zg = static_cast<const uint16_t *>(p.z);
    uint16_t *yg = static_cast<uint16_t *>(p.y);

    // A operands: U_k^T rows (channels) x K (rank), per tap k, tile t, K chunk c.
    bf16x8 ua[W][2][RC];
    load_u_rows<W, RC>(U, R, D, d0, lane, ua);

    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    // streams over the wave's rows [nbeg, nend): lane offset inside a step
    // plus the step's offset
    const uint32_t act_step = (uint32_t)(16 * D * 2);
    const uint32_t z_step = (uint32_t)(16 * R * 2);
    const uint32_t xoff = chan_ok ? (uint32_t)((tok * D + cbase) * 2) : kFar;
    uint32_t zoff[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        const int r0 = 32 * c + 8 * q;
        zoff[c] = r0 < R ? (uint32_t)((tok * R + r0) * 2) : kFar;
    }
    const __amdgpu_buffer_rsrc_t rx = make_stream(xg + nbeg * D, (nend - nbeg) * D * 2);
    const __amdgpu_buffer_rsrc_t rz = make_stream(zg + nbeg * R, (nend - nbeg) * R * 2);
    const __amdgpu_buffer_rsrc_t ry = make_stream(yg + nbeg * D, (nend - nbeg) * D * 2);

    // prefetch cursor (wave-uniform): the step being fetched
    int fstep = 0;
    int64_t fpos = nbeg;
    auto fetch = [&](uint4 &xd, uint4 (&zd)[RC]) {
        xd = buf_load16(rx, xoff + (uint32_t)fstep * act_step);
        if constexpr (RVEC) {
#pragma unroll
            for (int c = 0; c < RC; ++c) zd[c] = buf_load16(rz, zoff[c] + (uint32_t)fstep * z_step);
        } else {
            const int64_t n = fpos + tok;
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const int r0 = 32 * c + 8 * q;
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = (n < nend && r0 + 2 * e < R) ? zg[n * R + r0 + 2 * e] : 0u;
                    const uint32_t hi = (n < nend && r0 + 2 * e + 1 < R) ? zg[n * R + r0 + 2 * e + 1] : 0u;
                    h[e] = lo | (hi << 16);
                }
                zd[c] = make_uint4(h[0], h[1], h[2], h[3]);
            }
        }
        fstep += 1;
        fpos += 16;
    };

    __shared__ uint32_t seq_words[kBlock / kWave][kSeqWords];
    StartBits<kSeqWords> starts;
    starts.build(seq_words[threadIdx.x >> 6], p.seq, p.N, nbeg - 32, lane);

    // Register ring of PF step slots.  Step s reads slot s % PF (its x and z)
    // and slot (s-1) % PF (the previous x, for the taps that reach back across
    // the step edge), then refills slot (s-1) % PF with step s + PF - 1: no
    // value is copied between registers, so a load only has to land when its
    // step is computed.
    uint4 xq[PF];
    uint4 zq[PF][RC];
#pragma unroll
    for (int i = 0; i < PF - 1; ++i) fetch(xq[i], zq[i]);
    xq[PF - 1] = zero4;  // step -1: only its last W-1 tokens are read
    {
        const int64_t n = nbeg - 16 + tok;
        if (n >= 0 && tok >= 16 - (W - 1) && chan_ok)
            xq[PF - 1] = *reinterpret_cast<const uint4 *>(xg + n * D + cbase);
    }

    int64_t nstep = nbeg;

    for (int s0 = 0; s0 < nsteps; s0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            constexpr int kPrevOff = PF - 1;
            const int ip = (i + kPrevOff) % PF;
            {  // steps past the range read zeros and store nothing (buffer bounds)
                floatx4 acc[W][2];
#pragma unroll
                for (int k = 0; k < W; ++k)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            ua[k][t][0], __builtin_bit_cast(bf16x8, zq[i][0]), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                        for (int c = 1; c < RC; ++c)
                            acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                ua[k][t][c], __builtin_bit_cast(bf16x8, zq[i][c]), acc[k][t], 0, 0, 0);
                    }

                const uint32_t xc[4] = {xq[i].x, xq[i].y, xq[i].z, xq[i].w};
                const uint32_t xpv[4] = {xq[ip].x, xq[ip].y, xq[ip].z, xq[ip].w};
                Shifted<W> xs;
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) xs.v[0][i2] = xc[i2];
                fill_shift<W, 1>(xs, xc, xpv);

                // sequence masking, only when a sequence starts inside the
                // step's reach: bit j of win <-> token nstep - (W-1) + j
                if constexpr (W > 1) {
                    const uint32_t win = __builtin_amdgcn_readfirstlane(starts.window(nstep - (W - 1)));
                    if (win & (((1u << (W + 14)) - 1u) << 1)) {
                        // starts among tokens n-W+2 .. n (n = nstep + tok)
                        const uint32_t sub = (win >> (tok + 1)) & ((1u << (W - 1)) - 1u);
                        const int nv = sub ? (W - 2) - (31 - __builtin_clz(sub)) : W - 1;
#pragma unroll
                        for (int k = 1; k < W; ++k)
                            if (k > nv)
#pragma unroll
                                for (int i2 = 0; i2 < 4; ++i2) xs.v[k][i2] = 0u;
                    }
                }

                float out[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int t = c >> 2, j = c & 3;
                    float a = __uint_as_float(((c & 1) ? (xc[c >> 1] & 0xffff0000u) : (xc[c >> 1] << 16)) & p.rmask);
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const uint32_t v = xs.v[k][c >> 1];
                        const float xk = (c & 1) ? bf16_hi(v) : bf16_lo(v);
                        a = __builtin_fmaf(acc[k][t][j], xk, a);
                    }
                    out[c] = a;
                }
                uint4 v;
                v.x = pack_bf16x2(out[0], out[1]);
                v.y = pack_bf16x2(out[2], out[3]);
                v.z = pack_bf16x2(out[4], out[5]);
                v.w = pack_bf16x2(out[6], out[7]);
                buf_store16(ry, xoff + (uint32_t)(s0 + i) * act_step, v);

                fetch(xq[ip], zq[ip]);  // step s0 + i + PF - 1
                nstep += 16;
            }
        }
    }
}

// Look-ahead shift inside a 16-lane row: lane i takes lane i+K of `cur`, and
// lanes i >= 16-K take lane i+K-16 of `next` (the following 16 tokens).

template <int W, int K>
__device__ __forceinline__ void fill_ahead(Shifted<W> &gs, const uint32_t (&cur)[4], const uint32_t (&next)[4]) {
    if constexpr (K < W) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gs.v[K][i] = shift_ahead_in_row<K>(cur[i], next[i]);
        fill_ahead<W, K + 1>(gs, cur, next);
    }
}




// Backward of the fused low-rank convolution, bf16.
//
// Block = 4 waves, one 32-channel slice each, walking the same token range
// in steps of 16 tokens (pairs of steps = 32 tokens for the token
// contraction of dU).  Per step and wave:
//   * w of tokens n+k (k < W) on the matrix cores, B operand = z rows n+k
//     read from a wave-private LDS ring of z rows (A = U_k^T in registers);
//   * dx = rho*g + sum_k w_k * g shifted ahead by k (DPP with the next step);
//   * dwc_k = g * x shifted back by k (DPP with the previous step), rounded
//     to bf16 -- it is directly the B operand of dz^T = U_k * dwc_k, whose A
//     operand (U_k, rank rows x channel K) is also kept in registers;
//   * dwc_k is staged in LDS and re-read transposed (lane = channel,
//     registers = tokens) as the A operand of dU_k^T += dwc_k^T * Z.
// x, dy and z stream through one buffer resource each (offset = lane place +
// step offset), into register rings refilled P steps ahead without copies.
// dz is summed over the block's 4 waves in LDS and added to an fp32
// accumulator with one atomic per (token, rank), converted to bf16 by a
// launch after the kernel.  dU stays in registers over the whole token range
// and is added to the fp32 output with coalesced atomics at the end.  One
// launch before the kernel zeroes dU and the accumulator.
// H = 2 (R <= 32, W <= 4) doubles the block to 8 waves: two token halves
// over the same 4 channel slices, 2 waves per SIMD as with two 4-wave
// blocks, whose dU tiles are summed in LDS before the flush (half the dU
// atomics).
constexpr bool bwd_two_per_simd(int W, int RC) { return RC == 1 && W <= 4; }

template <int W, int RC, int H>
struct BwdLds {
    static constexpr int RP = 32 * RC;           // padded rank
    static constexpr int PW = 72;                // bytes per token row of dwc^T (32 ch + pad, 8-aligned)
    static constexpr int PZ = 2 * RP + 8;        // bytes per z row
    static constexpr int PD = 4 * RP + 16;       // bytes per token row of dz partials
    static constexpr int kDwc = W * 32 * PW;
    // z ring: 4 steps of 16 rows, then a copy of the first step's rows, so
    // that rows slot*16 + j (j < 32) are contiguous for every slot
    static constexpr int kZ = 80 * PZ;
    // 8 waves per CU (R <= 32, W <= 4: registers and LDS fit) keep one buffer
    // of dz partials per wave and pay a second barrier per pair; otherwise
    // the buffer is doubled and the pairs alternate.
    static constexpr bool kTwoPerSimd = bwd_two_per_simd(W, RC);
    static constexpr int kBlocksPerCu = kTwoPerSimd ? 2 / H : 1;
    static constexpr int kDzBufs = kTwoPerSimd ? 1 : 2;
    static constexpr int kDz = kDzBufs * 32 * PD;  // the wave's dz partials of kDzBufs pairs
    static constexpr int kLoop = kDwc + kZ + kDz;
    static constexpr int kDuPitch = 32 * W + 1;        // floats per rank row of the staged dU tile
    static constexpr int kDuStage = RP * kDuPitch * 4; // dU tile staged for coalesced atomics
    static constexpr int kWave = (((kLoop > kDuStage ? kLoop : kDuStage) + 15) / 16) * 16;
    static constexpr int kBlock = 4 * H * kWave;
    // (with the sequence-start maps and, for the RoPE instances, 128 bytes per wave of rotation constants)
    static_assert(kBlocksPerCu * (kBlock + 4 * H * 4 * kSeqWords + 4 * H * 128) <= 160 * 1024,
                  "the blocks of a CU must fit the LDS");
};



// Whether the backward's walk may end after any 32-token pair rather than
// after a whole ring of prefetch steps.  Only the two-half, 16-byte z variant
// takes it: in the other instances the early exit makes the compiler spill
// (the R = 64 kernel ran twice as long), so they walk whole rings.
constexpr bool bwd_exact_walk(int H, bool RVEC) { return H == 2 && RVEC; }

// DZ false: dx and dU only (dz is then computed by the kernels of
// lowrank_dz.hip); the dz products, their LDS exchange and its barriers and
// atomics are left out.  ROPE: the layer is followed by the rotary embedding
// of channels below p.rot, so dy is first turned back (the transposed
// rotation, at each token's position in its sequence) as it enters the
// look-ahead ring, and rounded to bf16 like the other matrix-core operands.
template <int W, int RC, int P, bool RVEC, int H, bool DZ = true, bool ROPE = false>
__global__ __launch_bounds__(kBlock * H, (BwdLds<W, RC, H>::kBlocksPerCu)) void lr_bwd_mfma(LrParams p, int64_t nslices,
                                                                                         int64_t tok_per_half) {
    using L = BwdLds<W, RC, H>;
    constexpr int RT = 2 * RC;  // 16-row rank tiles
    static_assert(P % 4 == 0, "the register rings cover whole turns of the 4-slot z ring");
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBlock];
    __shared__ uint32_t seq_words[4 * H][kSeqWords];
    // ROPE with one token half (kCarry below): each wave's turn by 16
    // positions for its 4 chunks of 8 channels
    constexpr bool kCarry = ROPE && H == 1;
    __shared__ __align__(16) float rope_r16[kCarry ? 4 : 1][kCarry ? 32 : 1];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = wid & 3;  // channel slice of the block's group
    const int half = wid >> 2;  // token half (H == 2)
    const int64_t ngroups = (nslices + 3) / 4;
    const int64_t tchunk = blockIdx.x / ngroups;
    const int64_t group = blockIdx.x - tchunk * ngroups;
    const int64_t d0 = (group * 4 + slice) * 32;
    const int64_t bbeg = tchunk * H * tok_per_half;  // the block's first token
    const int64_t nbeg = bbeg + half * tok_per_half;
    const int64_t nend = min(nbeg + tok_per_half, p.N);  // may be <= nbeg in the last block's second half
    // steps of both halves, from the first half's range, so all waves meet the
    // same barriers (steps past nend read zeros past N, store nothing past
    // nend, and add nothing to dz or dU): whole 32-token pairs when the walk
    // may end inside a ring (kExactWalk), else whole rings of P steps
    constexpr bool kExactWalk = bwd_exact_walk(H, RVEC);
    const int64_t len0 = min(tok_per_half, p.N - bbeg);
    const int64_t nsteps = kExactWalk ? ((len0 + 31) / 32) * 2 : ((len0 + 16 * P - 1) / (16 * P)) * P;

    const int tok = lane & 15;
    const int q = lane >> 4;
    const int i16 = lane & 15;
    const int64_t cbase = d0 + 8 * q;
    const bool chan_ok = cbase < p.D;
    const int R = p.R;
    const int64_t N = p.N;
    const int64_t D = p.D;
    const int64_t DW = D * W;

    const uint16_t *xg = static_cast<const uint16_t *>(p.x);
    const uint16_t *gg = static_cast<const uint16_t *>(p.dy);
    const uint16_t *zg = static_cast<const uint16_t *>(p.z);
    const uint16_t *U = static_cast<const uint16_t *>(p.U);
    uint16_t *dxg = static_cast<uint16_t *>(p.dx);

    unsigned char *my = lds + wid * L::kWave;
    unsigned char *dwcT = my;                       // [k][32 tokens][PW]
    unsigned char *zring = my + L::kDwc;            // [64 + 16 rows][PZ]
    unsigned char *dzb = my + L::kDwc + L::kZ;      // [32 tokens][PD]

    // ---- U operands, kept in registers for the whole walk
    bf16x8 ua[W][2][RC];  // rows: channel d0 + 8(i>>2) + 4t + (i&3); K: rank 32c + 8(lane>>4) + e
    bf16x8 ub[DZ ? W : 1][DZ ? RT : 1];  // rows: rank 16rt + (lane&15); K: channel d0 + 8(lane>>4) + e
    load_u_rows<W, RC>(U, R, D, d0, lane, ua);
    if constexpr (DZ) load_u_cols<W, RT>(U, R, D, d0, lane, ub);
    floatx4 du[W][2][RT];
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) du[k][ct][rt] = floatx4{0.f, 0.f, 0.f, 0.f};

    StartBits<kSeqWords> starts;
    starts.build(seq_words[wid], p.seq, N, nbeg - 32, lane);
    SeqPos sp{0};
    if constexpr (ROPE) {
        int64_t s_, e_;
        p.seq.find(nbeg < N ? nbeg : N - 1, s_, e_);
        sp.start = s_;
    }

    // ---- streams over the block's rows (x, dy and z up to N, dx up to nend):
    // lane offset inside a step plus the step's offset
    const uint32_t act_step = (uint32_t)(16 * D * 2);
    const uint32_t z_step = (uint32_t)(16 * R * 2);
    const uint32_t xoff = chan_ok ? (uint32_t)((tok * D + cbase) * 2) : kFar;
    uint32_t zoff[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        const int r0 = 32 * c + 8 * q;
        zoff[c] = r0 < R ? (uint32_t)((tok * R + r0) * 2) : kFar;
    }
    const __amdgpu_buffer_rsrc_t rx = make_stream(xg + nbeg * D, (N - nbeg) * D * 2);
    const __amdgpu_buffer_rsrc_t rg = make_stream(gg + nbeg * D, (N - nbeg) * D * 2);
    const __amdgpu_buffer_rsrc_t rz = make_stream(zg + nbeg * R, (N - nbeg) * R * 2);
    const __amdgpu_buffer_rsrc_t rdx = make_stream(dxg + nbeg * D, (nend - nbeg) * D * 2);
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    auto fetch_x = [&](int64_t step) { return buf_load16<kLrNtX>(rx, xoff + (uint32_t)step * act_step); };
    auto fetch_g = [&](int64_t step) { return buf_load16<kLrNtG>(rg, xoff + (uint32_t)step * act_step); };
    auto fetch_z = [&](int64_t step, uint4 (&dst)[RC]) {
        if constexpr (RVEC) {
#pragma unroll
            for (int c = 0; c < RC; ++c) dst[c] = buf_load16(rz, zoff[c] + (uint32_t)step * z_step);
        } else {
            const int64_t t0 = nbeg + 16 * step;
            const int64_t n = t0 + tok;
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const int r0 = 32 * c + 8 * q;
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = (n < N && r0 + 2 * e < R) ? zg[n * R + r0 + 2 * e] : 0u;
                    const uint32_t hi = (n < N && r0 + 2 * e + 1 < R) ? zg[n * R + r0 + 2 * e + 1] : 0u;
                    h[e] = lo | (hi << 16);
                }
                dst[c] = make_uint4(h[0], h[1], h[2], h[3]);
            }
        }
    };
    // z rows of ring slot `slot` (= step mod 4, known after unrolling)
    auto zrows = [&](int slot) { return zring + 16 * slot * L::PZ; };
    auto write_z = [&](int slot, const uint4 (&v)[RC]) {
#pragma unroll
        for (int copy = 0; copy < (slot == 0 ? 2 : 1); ++copy) {
            unsigned char *row = zring + (16 * (slot + 4 * copy) + tok) * L::PZ;
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                uint2 *d = reinterpret_cast<uint2 *>(row + 2 * (32 * c + 8 * q));
                d[0] = make_uint2(v[c].x, v[c].y);
                d[1] = make_uint2(v[c].z, v[c].w);
            }
        }
    };

    // ---- register rings (slot = step mod P), refilled without copies:
    //   x: step s reads slots s, s-1, then refills s-1 with step s+P-1
    //   g: step s reads slots s, s+1, then refills s with step s+P
    //   z: step s writes slot s+1 to the LDS ring, then refills it with step s+1+P
    uint4 xr[P], gr[P];
    uint4 zr[P][RC];
#pragma unroll
    for (int j = 0; j < P - 1; ++j) xr[j] = fetch_x(j);
    xr[P - 1] = zero4;  // step -1: only its last W-1 tokens are read
    {
        const int64_t n = nbeg - 16 + tok;
        if (n >= 0 && n < N && tok >= 16 - (W - 1) && chan_ok)
            xr[P - 1] = *reinterpret_cast<const uint4 *>(xg + n * D + cbase);
    }
#pragma unroll
    for (int j = 0; j < P; ++j) gr[j] = fetch_g(j);
    // dy of the 16 tokens from nstep turned back at their positions (steps in
    // order).  With two token halves (8 waves, registers at the limit) cos,
    // sin are read from the table at each step; with one (kCarry) they are
    // carried from step to step (RopeCarry), the turn by 16 positions read
    // from the wave's LDS copy, which measured faster there (no table load in
    // steady state) but spills registers in the two-half instances.
    RopeCarry rc;
    if constexpr (kCarry) {
        if (tok == 0) {
            float t16[8];
            rope_cs<8>(p, 16, cbase, t16);
#pragma unroll
            for (int e = 0; e < 8; ++e) rope_r16[wid][8 * q + e] = t16[e];
        }
        wave_lds_fence();
    }
    auto turn_g = [&](uint4 &v, int64_t nstep) {
        if constexpr (ROPE) {
            const int64_t pos = sp.pos_and_advance(starts, nstep, tok);
            float cs[8];
            if constexpr (kCarry) {
                if (nstep == nbeg) {
                    rc.start(p, pos, cbase);
                } else {
                    float r16[8];
                    const float4 a = *reinterpret_cast<const float4 *>(&rope_r16[wid][8 * q]);
                    const float4 b = *reinterpret_cast<const float4 *>(&rope_r16[wid][8 * q + 4]);
                    r16[0] = a.x; r16[1] = a.y; r16[2] = a.z; r16[3] = a.w;
                    r16[4] = b.x; r16[5] = b.y; r16[6] = b.z; r16[7] = b.w;
                    rc.advance(p, pos, cbase, r16, rope_restart(starts, nstep));
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) cs[e] = rc.c[e];
            }
            if (chan_ok && cbase < p.rot) {
                if constexpr (!kCarry) rope_cs<8>(p, pos, cbase, cs);
                uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {  // pair i2 = the two halves of word i2, turned back
                    const float a = bf16_lo(w4[i2]), b = bf16_hi(w4[i2]);
                    const float c = cs[2 * i2], sn = cs[2 * i2 + 1];
                    w4[i2] = pack_bf16x2(a * c + b * sn, b * c - a * sn);
                }
                v = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        }
    };
    turn_g(gr[0], nbeg);
    {
        uint4 z0[RC];
        fetch_z(0, z0);
        write_z(0, z0);
    }
    fetch_z(P, zr[0]);
#pragma unroll
    for (int j = 1; j < P; ++j) fetch_z(j, zr[j]);

    // dz atomics: rank of this lane and its element offset inside a pair
    // (each half reduces its own 4 waves with its own 256 threads)
    const int hthread = (int)threadIdx.x & (kBlock - 1);
    const int dz_rank = hthread % L::RP;
    const uint32_t dz_block_off = (uint32_t)((hthread / L::RP) * R + dz_rank);
    const unsigned char *dz_half = lds + 4 * half * L::kWave + L::kDwc + L::kZ;  // this half's first wave

    int buf = 0;
    for (int64_t s0 = 0; s0 < nsteps; s0 += P) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int cur = i, prv = (i + P - 1) % P, nxt = (i + 1) % P;
            const int ps = i & 1;
            const int64_t s = s0 + i;
            const int64_t nstep = nbeg + 16 * s;
            const int64_t n = nstep + tok;

            turn_g(gr[nxt], nstep + 16);     // the next step's dy, used from this step on
            write_z((i + 1) & 3, zr[nxt]);  // the wave's own LDS ring
            // other lanes read these rows below: keep the compiler from moving
            // the reads above the writes (the wave's LDS operations execute in order)
            wave_lds_fence();
            fetch_z(s + 1 + P, zr[nxt]);

            // sequence masks: taps k <= back (dwc) and k < ahead (dx) stay in n's
            // sequence; bit j of win <-> token nstep - (W-1) + j.  A step with no
            // sequence start among its taps' tokens, inside the block's range, runs
            // a copy of the step without the masks (the test is wave-uniform).
            int back = W - 1, ahead = W;
            bool fast = nstep + 16 <= nend;
            if constexpr (W > 1) {
                const uint32_t win = __builtin_amdgcn_readfirstlane(starts.window(nstep - (W - 1)));
                fast = fast && ((win >> 1) & ((1u << (2 * W + 13)) - 1u)) == 0u;  // the bits sb, sa test below
                const uint32_t sb = (win >> (tok + 1)) & ((1u << (W - 1)) - 1u);  // starts in n-W+2 .. n
                back = sb ? (W - 2) - (31 - __builtin_clz(sb)) : W - 1;
                const uint32_t sa = (win >> (tok + W)) & ((1u << (W - 1)) - 1u);  // starts in n+1 .. n+W-1
                ahead = sa ? 1 + __builtin_ctz(sa) : W;
            }
            auto body = [&](auto mask_tag) {
            constexpr bool M = decltype(mask_tag)::value;  // apply the masks

            const uint32_t gc[4] = {gr[cur].x, gr[cur].y, gr[cur].z, gr[cur].w};
            const uint32_t gn[4] = {gr[nxt].x, gr[nxt].y, gr[nxt].z, gr[nxt].w};
            const uint32_t xc[4] = {xr[cur].x, xr[cur].y, xr[cur].z, xr[cur].w};
            const uint32_t xp[4] = {xr[prv].x, xr[prv].y, xr[prv].z, xr[prv].w};

            // dx = rho*g + sum_k w[n+k] * g[n+k]; w of tokens n+k on the matrix cores,
            // rho entering as the accumulator of tap 0: dx = (w_0 + rho) g + sum_{k>0} ...
            float acc[8];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int rr = tok + k;
                const unsigned char *zrow = zrows(i & 3) + rr * L::PZ;
                bf16x8 zb[RC];
#pragma unroll
                for (int c = 0; c < RC; ++c) {
                    const uint2 *src = reinterpret_cast<const uint2 *>(zrow + 2 * (32 * c + 8 * q));
                    const uint2 a = src[0], b = src[1];
                    zb[c] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
                }
                uint32_t gk[4];
                if (k == 0) {
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) gk[i2] = gc[i2];
                } else {
                    shift_ahead4<W>(k, gc, gn, gk);
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) gk[i2] = (!M || k < ahead) ? gk[i2] : 0u;  // m+k in m's sequence
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const float c0 = k == 0 ? p.rho : 0.f;
                    floatx4 cw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[k][t][0], zb[0], floatx4{c0, c0, c0, c0},
                                                                         0, 0, 0);
#pragma unroll
                    for (int c = 1; c < RC; ++c)
                        cw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[k][t][c], zb[c], cw, 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = 4 * t + j;
                        const float gv = (c & 1) ? bf16_hi(gk[c >> 1]) : bf16_lo(gk[c >> 1]);
                        acc[c] = k == 0 ? cw[j] * gv : __builtin_fmaf(cw[j], gv, acc[c]);
                    }
                }
            }
            {
                uint4 v;
                v.x = pack_bf16x2(acc[0], acc[1]);
                v.y = pack_bf16x2(acc[2], acc[3]);
                v.z = pack_bf16x2(acc[4], acc[5]);
                v.w = pack_bf16x2(acc[6], acc[7]);
                buf_store16<kLrNtDx>(rdx, xoff + (uint32_t)s * act_step, v);
            }

            // dwc_k = g * x[n-k] (bf16): dz^T partial on the matrix cores, dwc^T staged for dU
            const bool own = n < nend;  // tokens outside this block's range contribute nothing
            floatx4 cz[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) cz[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < W; ++k) {
                uint32_t xk[4];
                if (k == 0) {
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) xk[i2] = xc[i2];
                } else {
                    shift_back4<W>(k, xc, xp, xk);
                }
                uint32_t dw[4];
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {
                    const uint32_t xv = (!M || (own && k <= back)) ? xk[i2] : 0u;
                    dw[i2] = pack_bf16x2(bf16_lo(gc[i2]) * bf16_lo(xv), bf16_hi(gc[i2]) * bf16_hi(xv));
                }
                const bf16x8 b = bf16x8_from_u32(dw);
                if constexpr (DZ) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        cz[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ub[k][rt], b, cz[rt], 0, 0, 0);
                }
                uint2 *d = reinterpret_cast<uint2 *>(dwcT + k * 32 * L::PW + (16 * ps + tok) * L::PW + 16 * q);
                d[0] = make_uint2(dw[0], dw[1]);
                d[1] = make_uint2(dw[2], dw[3]);
            }
            // dz partials (rows r = 16rt + 4q + j, column = token) -> LDS for the block reduction
            if constexpr (DZ) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    float4 *d =
                        reinterpret_cast<float4 *>(dzb + (buf * 32 + 16 * ps + tok) * L::PD + 4 * (16 * rt + 4 * q));
                    *d = make_float4(cz[rt][0], cz[rt][1], cz[rt][2], cz[rt][3]);
                }
            }
            };
            if (fast) body(MaskTag<false>{}); else body(MaskTag<true>{});

            // ring refills (issued after the step's reads of these slots)
            xr[prv] = fetch_x(s + P - 1);
            gr[cur] = fetch_g(s + P);

            if (ps == 1) {
                if constexpr (DZ) {
                    lds_barrier();  // the pair's dz partials from all four waves
                } else {
                    wave_lds_fence();  // the pair's dwc^T rows written by the wave's other lanes
                }
                // dU_k^T[ch, r] += sum over the pair's 32 tokens of dwc_k^T[ch, tok] * z[tok, r].
                // Operands re-read transposed from LDS: lane = channel / rank,
                // registers = tokens 8q .. 8q+7 of the pair.
                const int64_t s_pair = s - 1;
                const int trow = 8 * q + (i16 >> 2);  // row addressed by this lane (first half)
                const int tcol = 4 * (i16 & 3);        // column chunk addressed by this lane
                bf16x8 zb[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    uint2 h[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int row = trow + 4 * hh;
                        h[hh] = lds_read_tr(zrows((i - 1) & 3) + row * L::PZ + 2 * (16 * rt + tcol));
                    }
                    zb[rt] = __builtin_bit_cast(bf16x8, make_uint4(h[0].x, h[0].y, h[1].x, h[1].y));
                }
#pragma unroll
                for (int k = 0; k < W; ++k) {
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        uint2 h[2];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            h[hh] = lds_read_tr(dwcT + k * 32 * L::PW + (trow + 4 * hh) * L::PW + 2 * (16 * ct + tcol));
                        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(h[0].x, h[0].y, h[1].x, h[1].y));
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            du[k][ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, zb[rt], du[k][ct][rt], 0, 0, 0);
                    }
                }

                // dz of the pair's 32 tokens: fp32 atomics into the accumulator, issued
                // only by lanes of ranks below R and tokens inside the block's range,
                // each at an in-range offset of a resource based at the pair's row
                if constexpr (DZ) {
                const int64_t npair0 = nbeg + 16 * s_pair;
                const __amdgpu_buffer_rsrc_t rdz =
                    make_stream(p.dzacc + group * p.dz_gstride + npair0 * R, (nend - npair0) * R * 4);
                {
                    // per half: thread e sums (token e / RP, rank e % RP) over the half's four waves
                    constexpr int kIt = 32 * L::RP / kBlock;
                    float v[kIt];
#pragma unroll
                    for (int it = 0; it < kIt; ++it) {
                        const int e = hthread + it * kBlock, tl = e / L::RP, r = e % L::RP;
                        const unsigned char *src = dz_half + (buf * 32 + tl) * L::PD + 4 * r;
                        float a = 0.f;
#pragma unroll
                        for (int w2 = 0; w2 < 4; ++w2) a += *reinterpret_cast<const float *>(src + w2 * L::kWave);
                        v[it] = a;
                    }
#pragma unroll
                    for (int it = 0; it < kIt; ++it) {
                        const int tl = hthread / L::RP + it * (kBlock / L::RP);
                        if (dz_rank < R && npair0 + tl < nend)
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                                v[it], rdz, 4 * (dz_block_off + (uint32_t)(it * (kBlock / L::RP) * R)), 0, 0);
                    }
                    if constexpr (L::kDzBufs == 1) {
                        lds_barrier();  // partials read before the next pair overwrites them
                    } else {
                        buf ^= 1;         // the next pair writes the other buffer
                    }
                }
                }
            }
            if constexpr (kExactWalk) {
                if (ps == 1 && s + 1 >= nsteps) break;  // the walk's last pair (block-uniform)
            }
        }
    }

    // dU tile of this wave (rank x 32 channels x W taps) -> LDS in the memory
    // order of dU (odd row pitch, so a wave's staging writes spread over the
    // banks), then added to the output with coalesced atomics: each wave
    // instruction covers 64 consecutive floats of one rank row.  Every wave
    // flushes ranks of its own slice; with H == 2 the two halves take
    // alternate groups of 4 ranks and add both halves' tiles.
    __syncthreads();  // every wave is done with the loop's LDS regions
    constexpr int kPitch = L::kDuPitch;
    float *dus = reinterpret_cast<float *>(my);
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int r = 16 * rt + i16;
#pragma unroll
                for (int j = 0; j < 4; ++j) dus[r * kPitch + (16 * ct + 4 * q + j) * W + k] = du[k][ct][rt][j];
            }
    __syncthreads();
    {
        const float *t0 = reinterpret_cast<const float *>(lds + slice * L::kWave);
        const float *t1 = reinterpret_cast<const float *>(lds + (4 + slice) * L::kWave);  // read only with H == 2
        const int nvalid = (int)((D - d0 < 32 ? D - d0 : 32) * W);  // floats of this slice inside D
        constexpr int kJ = (32 * W + kWave - 1) / kWave;
        float *dst = p.dU + tchunk * p.du_cstride + d0 * W;
        // ranks rb .. rb+3 stay below RP (rb is a multiple of 4 below R <= RP, and
        // RP is a multiple of 32): the tile reads are in bounds; ranks >= R are
        // not added
#pragma unroll 1
        for (int rb = 4 * half; rb < R; rb += 4 * H) {
            float v[4][kJ];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    const int idx = lane + kWave * j;
                    float a = 0.f;
                    if (idx < 32 * W) {
                        a = t0[(rb + u) * kPitch + idx];
                        if constexpr (H == 2) a += t1[(rb + u) * kPitch + idx];
                    }
                    v[u][j] = a;
                }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    const int idx = lane + kWave * j;
                    if (rb + u < R && idx < nvalid) atomicAdd(dst + (int64_t)(rb + u) * DW + idx, v[u][j]);
                }
        }
    }
}

// ------------------------------------------------------------ small kernels

__global__ void fill_zero_f32(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// Zeroes two 16-byte aligned arrays of 32-bit words in one launch; thread
// i clears words 4i .. 4i+3 of the concatenation (vector store when whole).
__device__ __forceinline__ void zero_words(uint32_t *p, int64_t n, int64_t unit) {
    const int64_t i = 4 * unit;
    if (i + 3 < n) {
        *reinterpret_cast<uint4 *>(p + i) = make_uint4(0u, 0u, 0u, 0u);
    } else {
        for (int64_t j = i; j < n; ++j) p[j] = 0u;
    }
}

__global__ void clear2(uint32_t *a, int64_t na, uint32_t *b, int64_t nb) {
    int64_t u = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t ua = (na + 3) / 4, ub = (nb + 3) / 4;
    if (u < ua) return zero_words(a, na, u);
    u -= ua;
    if (u < ub) zero_words(b, nb, u);
}

__global__ void cast_f32_bf16(const float *src, uint16_t *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) dst[i] = to_bf16(src[i]);
}

// ------------------------------------------- deterministic split-K sums
//
// The reproducible backward (dsc_lowrank_bwd_deterministic) forms every sum
// in one fixed order.  The matrix-core kernel then adds the dz of each
// channel group and the dU of each token chunk into regions of their own,
// zeroed first, that receive exactly one term per element (so each value is
// exact); these kernels add the regions in ascending order.  The generic
// kernels' atomics are replaced by one thread per dz or dU element.

template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return to_bf16(v); }

// dst[i] = src[i] + src[stride + i] + ... + src[(nparts-1)*stride + i], in that order.
template <class T>
__global__ __launch_bounds__(kBlock) void sum_parts(const float *src, int64_t nparts, int64_t stride, T *dst,
                                                    int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    float a = 0.f;
    // unrolled so that the loads of several regions are in flight together; the
    // additions keep the ascending order
#pragma unroll 16
    for (int64_t j = 0; j < nparts; ++j) a += src[j * stride + i];
    dst[i] = from_f32<T>(a);
}

// dz[n,r] = sum over channels d, then taps k (ascending) of U[r,d*W+k] * dwc[n,d,k].
template <class E, int W>
__global__ __launch_bounds__(kBlock) void lr_dz_direct(LrParams p) {
    using S = typename E::store_t;
    const int64_t item = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (item >= p.N * p.R) return;
    const int64_t n = item / p.R;
    const int64_t r = item - n * p.R;
    const S *x = static_cast<const S *>(p.x);
    const S *g = static_cast<const S *>(p.dy);
    const S *U = static_cast<const S *>(p.U);
    int64_t s, e;
    p.seq.find(n, s, e);
    const int kn = (int)(n - s + 1 < W ? n - s + 1 : W);  // taps whose token n-k is in n's sequence
    float acc = 0.f;
    for (int64_t d = 0; d < p.D; ++d) {
        const float gv = load_elem<E>(g + n * p.D + d);
        const S *u = U + (r * p.D + d) * W;
        for (int k = 0; k < kn; ++k)
            acc = __builtin_fmaf(load_elem<E>(u + k), gv * load_elem<E>(x + (n - k) * p.D + d), acc);
    }
    static_cast<S *>(p.dz)[item] = from_f32<S>(acc);
}

// dU[r,d*W+k] = sum over tokens n (ascending) of z[n,r] * dwc[n,d,k], in
// partial sums of 256 tokens added in order.
template <class E, int W>
__global__ __launch_bounds__(kBlock) void lr_du_direct(LrParams p) {
    using S = typename E::store_t;
    const int64_t DW = p.D * W;
    const int64_t item = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (item >= p.R * DW) return;
    const int64_t r = item / DW;
    const int64_t d = (item - r * DW) / W;
    const int k = (int)(item - r * DW - d * W);
    const S *x = static_cast<const S *>(p.x);
    const S *g = static_cast<const S *>(p.dy);
    const S *z = static_cast<const S *>(p.z);
    float total = 0.f;
    int64_t s = 0, e = 0;  // sequence of the current token: [s, e)
    for (int64_t n0 = 0; n0 < p.N; n0 += 256) {
        const int64_t n1 = n0 + 256 < p.N ? n0 + 256 : p.N;
        float part = 0.f;
        for (int64_t n = n0; n < n1; ++n) {
            if (n >= e) p.seq.find(n, s, e);
            if (n - k >= s)
                part = __builtin_fmaf(load_elem<E>(z + n * p.R + r),
                                      load_elem<E>(g + n * p.D + d) * load_elem<E>(x + (n - k) * p.D + d), part);
        }
        total += part;
    }
    p.dU[item] = total;
}

template <class E, int W, bool ROPE = false>
hipError_t generic_fwd(const LrProblem &pr, hipStream_t st) {
    LrParams p = make_params<E>(pr);
    const int64_t b = nblocks(p.N * p.nchunks);
    if (b) hipLaunchKernelGGL((lr_fwd_generic<E, W, ROPE>), dim3((unsigned)b), dim3(kBlock), 0, st, p);
    return hipGetLastError();
}

// dx, then dz and dU one thread per element (fixed order, no workspace).
template <class E, int W>
hipError_t generic_bwd_det(const LrProblem &pr, hipStream_t st) {
    LrParams p = make_params<E>(pr);
    const int64_t b = nblocks(p.N * p.nchunks);
    if (b) hipLaunchKernelGGL((lr_bwd_generic<E, W, false>), dim3((unsigned)b), dim3(kBlock), 0, st, p);
    hipLaunchKernelGGL((lr_dz_direct<E, W>), dim3((unsigned)nblocks(p.N * p.R)), dim3(kBlock), 0, st, p);
    hipLaunchKernelGGL((lr_du_direct<E, W>), dim3((unsigned)nblocks((int64_t)p.R * p.D * W)), dim3(kBlock), 0, st, p);
    return hipGetLastError();
}

template <class E, int W, bool ROPE = false>
hipError_t generic_bwd(const LrProblem &pr, hipStream_t st, bool det = false) {
    if constexpr (!ROPE) {
        if (det) return generic_bwd_det<E, W>(pr, st);
    }
    LrParams p = make_params<E>(pr);
    const int64_t nU = (int64_t)p.R * p.D * W;
    const int64_t nz = p.N * p.R;
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)nblocks(nU)), dim3(kBlock), 0, st, p.dU, nU);
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, p.dzacc, nz);
    const int64_t b = nblocks(p.N * p.nchunks);
    if (b) hipLaunchKernelGGL((lr_bwd_generic<E, W, true, ROPE>), dim3((unsigned)b), dim3(kBlock), 0, st, p);
    if constexpr (sizeof(typename E::store_t) == 2)
        hipLaunchKernelGGL(cast_f32_bf16, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, p.dzacc,
                           static_cast<uint16_t *>(p.dz), nz);
    return hipGetLastError();
}

#ifndef DSC_LR_FWD_WAVES
#define DSC_LR_FWD_WAVES 3072
#endif
// Forward (R > 32) tuning, measured on MI355X: the prefetch ring depth in
// 16-token steps and the number of waves the grid aims for.  These kernels
// stay bandwidth-bound with a partly filled last round, so the grid is not
// cut to one round of resident waves.
template <int RC>
struct FwdTune {
    static constexpr int kPF = RC == 1 ? 8 : 6;
    static constexpr int64_t kWaves = DSC_LR_FWD_WAVES;
};

template <int W, int RC>
hipError_t mfma_fwd(const LrProblem &pr, hipStream_t st) {
    constexpr int PF = FwdTune<RC>::kPF;
    LrParams p = make_params<BF16>(pr);
    const int64_t nslices = (p.D + 31) / 32;
    const int64_t cap = walk_cap(p.D, 16 * PF, 16 * (2 * PF + 2));
    if (cap < 16 * PF) return generic_fwd<BF16, W>(pr, st);
    int64_t tpw = (p.N * nslices + FwdTune<RC>::kWaves - 1) / FwdTune<RC>::kWaves;
    tpw = ((tpw + 16 * PF - 1) / (16 * PF)) * (16 * PF);  // whole groups of PF steps
    if (tpw > cap) tpw = cap;
    const bool rvec = p.R % 8 == 0;
    const int64_t waves = ((p.N + tpw - 1) / tpw) * nslices;
    const int64_t b = (waves + 3) / 4;
    if (b) {
        if (rvec)
            hipLaunchKernelGGL((lr_fwd_mfma<W, RC, PF, true>), dim3((unsigned)b), dim3(kBlock), 0, st, p, nslices, tpw);
        else
            hipLaunchKernelGGL((lr_fwd_mfma<W, RC, PF, false>), dim3((unsigned)b), dim3(kBlock), 0, st, p, nslices, tpw);
    }
    return hipGetLastError();
}

#ifndef DSC_LR_BWD_RING
#define DSC_LR_BWD_RING 4
#endif
constexpr int kBwdRing = DSC_LR_BWD_RING;  // backward prefetch ring depth (steps)
constexpr int64_t kBlockFixedTokens = 256;  // a block's set-up and dU flush, in tokens of walk (measured)

// Work split of the matrix-core backward: H token halves per block, blocks
// of 4 channel slices (ngroups across D) and token chunks of 2 * tph tokens.
struct BwdPlan {
    int64_t ngroups, tph, tchunks;
};

BwdPlan bwd_plan(int64_t N, int64_t D, int W, int R, int64_t slots) {
    const int H = bwd_two_per_simd(W, (R + 31) / 32) ? 2 : 1;
    const int64_t cap = walk_cap(D, 16 * kBwdRing, 16 * (2 * kBwdRing + 2));
    const int64_t ngroups = ((D + 31) / 32 + 3) / 4;
    // walk unit: a 32-token pair per half where the walk may stop there, else a ring
    const int64_t unit = bwd_exact_walk(H, R % 8 == 0) ? H * 32 : H * 16 * kBwdRing;
    const int64_t block_len = walk_length(N, ngroups, slots, H * cap, unit, H * kBlockFixedTokens);
    return BwdPlan{ngroups, block_len / H, (N + block_len - 1) / block_len};
}

// Whether the bf16 backward of these sizes runs the matrix-core kernel: it
// keeps W*RC*(two U operand sets + dU tiles) in registers and is instantiated
// while that fits (W*RC <= 8); the walk cap must hold a ring.
bool bwd_uses_mfma(Dtype dt, int64_t D, int W, int R) {
    const int rc = (R + 31) / 32;
    if (dt != Dtype::BF16 || W < 1 || W > 8 || !(rc == 1 || (rc == 2 && W <= 4))) return false;
    return walk_cap(D, 16 * kBwdRing, 16 * (2 * kBwdRing + 2)) >= 16 * kBwdRing;
}


size_t det_dz_floats(const BwdPlan &pl, int64_t N, int R) { return (((size_t)pl.ngroups * N * R + 3) / 4) * 4; }

template <int W, int RC, bool ROPE = false>
hipError_t mfma_bwd(const LrProblem &pr, hipStream_t st, bool det) {
    LrParams p = make_params<BF16>(pr);
    const int64_t nU = (int64_t)p.R * p.D * W;
    const int64_t nz = p.N * p.R;
    constexpr int H = bwd_two_per_simd(W, RC) ? 2 : 1;  // token halves per block
    int64_t slots = kDetSlots;
    if (!det) {
        static const int bpc_vec = blocks_per_cu(
            reinterpret_cast<const void *>(&lr_bwd_mfma<W, RC, kBwdRing, true, H, true, ROPE>), kBlock * H);
        static const int bpc_gather = blocks_per_cu(
            reinterpret_cast<const void *>(&lr_bwd_mfma<W, RC, kBwdRing, false, H, true, ROPE>), kBlock * H);
        slots = (int64_t)device_cus() * (p.R % 8 == 0 ? bpc_vec : bpc_gather);
    }
    const BwdPlan pl = bwd_plan(p.N, p.D, W, p.R, slots);
    float *dz_sum = p.dzacc, *du_sum = p.dU;
    int64_t nclear_dz = nz, nclear_du = nU;
    if (det) {  // regions of their own: dz per channel group, dU per token chunk
        p.dz_gstride = nz;
        p.du_cstride = nU;
        p.dU = p.dzacc + det_dz_floats(pl, p.N, p.R);
        nclear_dz = pl.ngroups * nz;
        nclear_du = pl.tchunks * nU;
    }
    // one launch clears dU and the dz accumulator (or their regions)
    const int64_t units = (nclear_du + 3) / 4 + (nclear_dz + 3) / 4;
    hipLaunchKernelGGL(clear2, dim3((unsigned)nblocks(units)), dim3(kBlock), 0, st,
                       reinterpret_cast<uint32_t *>(p.dU), nclear_du, reinterpret_cast<uint32_t *>(p.dzacc), nclear_dz);
    const dim3 grid((unsigned)(pl.tchunks * pl.ngroups));
    const int64_t nslices = (p.D + 31) / 32;
    if (p.R % 8 == 0)
        hipLaunchKernelGGL((lr_bwd_mfma<W, RC, kBwdRing, true, H, true, ROPE>), grid, dim3(kBlock * H), 0, st, p,
                           nslices, pl.tph);
    else
        hipLaunchKernelGGL((lr_bwd_mfma<W, RC, kBwdRing, false, H, true, ROPE>), grid, dim3(kBlock * H), 0, st, p,
                           nslices, pl.tph);
    if (det) {
        hipLaunchKernelGGL(sum_parts<uint16_t>, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, dz_sum,
                           pl.ngroups, nz, static_cast<uint16_t *>(pr.dz), nz);
        hipLaunchKernelGGL(sum_parts<float>, dim3((unsigned)nblocks(nU)), dim3(kBlock), 0, st, p.dU, pl.tchunks, nU,
                           du_sum, nU);
    } else {
        hipLaunchKernelGGL(cast_f32_bf16, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, p.dzacc,
                           static_cast<uint16_t *>(p.dz), nz);
    }
    return hipGetLastError();
}

// Which bf16 shapes compute dz in launches of their own (split backward):
// the matrix-core backward then runs without dz, so its blocks exchange
// nothing and add no dz atomics.
// Whether ranks 33..64 at W = 2..4 take the backward with each 32-channel
// slice split between two waves by channels (lowrank_taps.hip).
#ifndef DSC_LR_TAPS
#define DSC_LR_TAPS 1
#endif

#ifndef DSC_LR_SPLIT
#define DSC_LR_SPLIT 0
#endif
bool bwd_split(Dtype dt, int64_t D, int W, int R) {
    if (!bwd_uses_mfma(dt, D, W, R) || !lowrank_dz_supported(W, R)) return false;
    if (DSC_LR_SPLIT == 2) return true;
    return DSC_LR_SPLIT == 1 && (R + 31) / 32 == 2;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t split_workspace(int64_t N, int64_t D, int W, int R) {
    const LrDzPlan pl = lowrank_dz_plan(N, D, W, R);
    return align256((size_t)pl.ut_elems * 2) + align256((size_t)pl.part_floats * 4);
}

// dx and dU from the matrix-core kernel without dz; dz from the kernels of
// lowrank_dz.hip into the workspace ([tap-major U][partials per channel
// split]), then the partials added in order and rounded to bf16.
template <int W, int RC>
hipError_t split_bwd(const LrProblem &pr, hipStream_t st) {
    LrParams p = make_params<BF16>(pr);
    const int64_t nU = (int64_t)p.R * p.D * W;
    const int64_t nz = p.N * p.R;
    constexpr int H = bwd_two_per_simd(W, RC) ? 2 : 1;
    static const int bpc_vec = blocks_per_cu(
        reinterpret_cast<const void *>(&lr_bwd_mfma<W, RC, kBwdRing, true, H, false>), kBlock * H);
    static const int bpc_gather = blocks_per_cu(
        reinterpret_cast<const void *>(&lr_bwd_mfma<W, RC, kBwdRing, false, H, false>), kBlock * H);
    const int64_t slots = (int64_t)device_cus() * (p.R % 8 == 0 ? bpc_vec : bpc_gather);
    const BwdPlan pl = bwd_plan(p.N, p.D, W, p.R, slots);
    const LrDzPlan dzp = lowrank_dz_plan(p.N, p.D, W, p.R);
    unsigned char *ws = reinterpret_cast<unsigned char *>(pr.dz_acc);
    uint16_t *Ut = reinterpret_cast<uint16_t *>(ws);
    float *parts = reinterpret_cast<float *>(ws + align256((size_t)dzp.ut_elems * 2));
    hipLaunchKernelGGL(clear2, dim3((unsigned)nblocks((nU + 3) / 4)), dim3(kBlock), 0, st,
                       reinterpret_cast<uint32_t *>(p.dU), nU, static_cast<uint32_t *>(nullptr), (int64_t)0);
    const dim3 grid((unsigned)(pl.tchunks * pl.ngroups));
    const int64_t nslices = (p.D + 31) / 32;
    if (p.R % 8 == 0)
        hipLaunchKernelGGL((lr_bwd_mfma<W, RC, kBwdRing, true, H, false>), grid, dim3(kBlock * H), 0, st, p, nslices,
                           pl.tph);
    else
        hipLaunchKernelGGL((lr_bwd_mfma<W, RC, kBwdRing, false, H, false>), grid, dim3(kBlock * H), 0, st, p,
                           nslices, pl.tph);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = lowrank_dz_partials(pr, dzp, Ut, parts, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sum_parts<uint16_t>, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, parts,
                       (int64_t)dzp.S, nz, static_cast<uint16_t *>(pr.dz), nz);
    return hipGetLastError();
}

template <int W>
hipError_t mfma_bwd_rc(const LrProblem &pr, hipStream_t st, bool det, bool split_ok = true) {
    if (!bwd_uses_mfma(Dtype::BF16, pr.D, W, pr.R)) return generic_bwd<BF16, W>(pr, st, det);
    if (!det && split_ok && bwd_split(Dtype::BF16, pr.D, W, pr.R)) {
        if constexpr (W <= 4) {
            if ((pr.R + 31) / 32 == 2) return split_bwd<W, 2>(pr, st);
        }
        return split_bwd<W, 1>(pr, st);
    }
    if constexpr (W <= 4) {
        if ((pr.R + 31) / 32 == 2) {
            if (DSC_LR_TAPS && lowrank_bwd_taps_supported(Dtype::BF16, pr.D, W, pr.R))
                return lowrank_bwd_taps(pr, st, det);
            return mfma_bwd<W, 2>(pr, st, det);
        }
    }
    return mfma_bwd<W, 1>(pr, st, det);
}

template <int W>
hipError_t mfma_fwd_rc(const LrProblem &pr, hipStream_t st) {
    switch ((pr.R + 31) / 32) {
        case 1: return mfma_fwd<W, 1>(pr, st);
        case 2: return mfma_fwd<W, 2>(pr, st);
        case 3: return mfma_fwd<W, 3>(pr, st);
        case 4: return mfma_fwd<W, 4>(pr, st);
        default: return hipErrorInvalidValue;
    }
}

// The layer followed by the rotary embedding: the wide forward (R <= 64) or
// the generic one; the fused matrix-core backward (dz in the same kernel, no
// split) where it runs, else the generic one.
template <int W>
hipError_t rope_fwd_w(const LrProblem &pr, hipStream_t st) {
    if (pr.dtype == Dtype::BF16) {
        bool used = false;
        const hipError_t e = lowrank_fwd_wide(pr, st, &used);
        if (used) return e;
        return generic_fwd<BF16, W, true>(pr, st);
    }
    return generic_fwd<F32, W, true>(pr, st);
}

template <int W>
hipError_t rope_bwd_w(const LrProblem &pr, hipStream_t st) {
    if (pr.dtype == Dtype::F32) return generic_bwd<F32, W, true>(pr, st);
    if (!bwd_uses_mfma(Dtype::BF16, pr.D, W, pr.R)) return generic_bwd<BF16, W, true>(pr, st);
    if constexpr (W <= 4) {
        if ((pr.R + 31) / 32 == 2) {
            if (DSC_LR_TAPS && lowrank_bwd_taps_supported(Dtype::BF16, pr.D, W, pr.R))
                return lowrank_bwd_taps_rope(pr, st);
            return mfma_bwd<W, 2, true>(pr, st, false);
        }
    }
    return mfma_bwd<W, 1, true>(pr, st, false);
}

#define DSC_W_SWITCH(W_, CALL)             \
    switch (W_) {                          \
        case 1: { constexpr int Wc = 1; return CALL; } \
        case 2: { constexpr int Wc = 2; return CALL; } \
        case 3: { constexpr int Wc = 3; return CALL; } \
        case 4: { constexpr int Wc = 4; return CALL; } \
        case 5: { constexpr int Wc = 5; return CALL; } \
        case 6: { constexpr int Wc = 6; return CALL; } \
        case 7: { constexpr int Wc = 7; return CALL; } \
        case 8: { constexpr int Wc = 8; return CALL; } \
        default: return hipErrorInvalidValue; \
    }

}  // namespace

size_t lowrank_bwd_workspace(Dtype dt, int64_t N, int64_t D, int32_t W, int32_t R, bool split_ok) {
    if (dt == Dtype::F32) return 0;
    if (split_ok && bwd_split(dt, D, W, R)) return split_workspace(N, D, W, R);
    const size_t bytes = (size_t)N * (size_t)R * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t lowrank_fwd(const LrProblem &p, hipStream_t s) {
    if (p.dtype == Dtype::BF16) {
        bool used = false;
        const hipError_t e = lowrank_fwd_wide(p, s, &used);  // R <= 64 (lowrank_fwd.hip)
        if (used) return e;
        DSC_W_SWITCH(p.W, mfma_fwd_rc<Wc>(p, s));
    }
    DSC_W_SWITCH(p.W, (generic_fwd<F32, Wc>(p, s)));
}

hipError_t lowrank_zero(float *p, int64_t n, hipStream_t s) {
    const int64_t units = (n + 3) / 4;
    if (units) hipLaunchKernelGGL(clear2, dim3((unsigned)nblocks(units)), dim3(kBlock), 0, s,
                                  reinterpret_cast<uint32_t *>(p), n, static_cast<uint32_t *>(nullptr), (int64_t)0);
    return hipGetLastError();
}

hipError_t lowrank_zero2(float *a, int64_t na, float *b, int64_t nb, hipStream_t s) {
    const int64_t units = (na + 3) / 4 + (nb + 3) / 4;
    if (units) hipLaunchKernelGGL(clear2, dim3((unsigned)nblocks(units)), dim3(kBlock), 0, s,
                                  reinterpret_cast<uint32_t *>(a), na, reinterpret_cast<uint32_t *>(b), nb);
    return hipGetLastError();
}

hipError_t lowrank_sum_parts(const float *src, int64_t nparts, int64_t stride, float *dst_f32, uint16_t *dst_bf16,
                             int64_t n, hipStream_t s) {
    if (!n) return hipSuccess;
    if (dst_bf16)
        hipLaunchKernelGGL(sum_parts<uint16_t>, dim3((unsigned)nblocks(n)), dim3(kBlock), 0, s, src, nparts, stride,
                           dst_bf16, n);
    else
        hipLaunchKernelGGL(sum_parts<float>, dim3((unsigned)nblocks(n)), dim3(kBlock), 0, s, src, nparts, stride,
                           dst_f32, n);
    return hipGetLastError();
}

hipError_t lowrank_round_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t s) {
    if (n) hipLaunchKernelGGL(cast_f32_bf16, dim3((unsigned)nblocks(n)), dim3(kBlock), 0, s, src, dst, n);
    return hipGetLastError();
}

hipError_t lowrank_bwd(const LrProblem &p, hipStream_t s, bool split_ok) {
    if (p.dtype == Dtype::BF16) {
        DSC_W_SWITCH(p.W, (mfma_bwd_rc<Wc>(p, s, false, split_ok)));
    }
    DSC_W_SWITCH(p.W, (generic_bwd<F32, Wc>(p, s)));
}

size_t lowrank_bwd_det_workspace(Dtype dt, int64_t N, int64_t D, int32_t W, int32_t R) {
    if (!bwd_uses_mfma(dt, D, W, R)) return 0;
    if (DSC_LR_TAPS && lowrank_bwd_taps_supported(dt, D, W, R)) return lowrank_bwd_taps_det_workspace(N, D, W, R);
    const BwdPlan pl = bwd_plan(N, D, W, R, kDetSlots);
    const size_t bytes = (det_dz_floats(pl, N, R) + (size_t)pl.tchunks * R * D * W) * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t lowrank_rope_fwd(const LrProblem &p, hipStream_t s) {
    if (p.rot <= 0) return lowrank_fwd(p, s);
    DSC_W_SWITCH(p.W, rope_fwd_w<Wc>(p, s));
}

hipError_t lowrank_rope_bwd(const LrProblem &p, hipStream_t s) {
    if (p.rot <= 0) return lowrank_bwd(p, s, false);
    DSC_W_SWITCH(p.W, rope_bwd_w<Wc>(p, s));
}

hipError_t lowrank_bwd_det(const LrProblem &p, hipStream_t s) {
    if (p.dtype == Dtype::BF16) {
        DSC_W_SWITCH(p.W, (mfma_bwd_rc<Wc>(p, s, true)));
    }
    DSC_W_SWITCH(p.W, (generic_bwd<F32, Wc>(p, s, true)));
}

}  // namespace dsc
