// lowrank_dz.hip -- dz of the low-rank backward as a launch of its own, for
// gfx950 (bf16).
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: parametrization (1) low-rank factorisation
// w(t) = z_t U; the backward is the chain rule of the mechanism for
// L = <dy, y>):
//   dwc[n,d,k] = [n-k in seq(n)] dy[n,d] x[n-k,d]      (rounded to bf16)
//   dz[n,r]    = sum_{d,k} U[r, d*W+k] dwc[n,d,k]
// i.e. dz (N x R) = sum_k dwc_k (N x D) U_k^T (D x R): a matrix product whose
// left operand is formed on chip from dy and x, contracted over channels.
//
// Design:
//   * a wave owns MT tiles of 16 tokens (lane = token of a tile, four groups
//     of 8 channels), a block of 4 waves owns 64*MT consecutive tokens and one
//     range of channels (a split of D); every dz term of those tokens and
//     channels is summed on chip, in a fixed order, and each split writes its
//     fp32 partial sums to a region of its own (no atomics), which a second
//     launch adds in ascending order;
//   * per 32 channels: dy and x rows of the wave's tokens (16-byte vectors of
//     8 channels), the x of tap k shifted by k tokens with DPP row moves (the
//     first tile takes its W-1 earlier rows from a halo load); dwc_k is the B
//     operand of v_mfma_f32_16x16x32_bf16 and the 32-channel slice of U_k,
//     staged once per block in LDS (tap-major copy of U made beforehand), the
//     A operand: C = dz^T (ranks x tokens), 4 ranks of one token per lane;
//   * U and the next 32 channels of dy and x are fetched while the current
//     ones are multiplied (U through a double-buffered LDS slice);
//   * taps that reach before a token's sequence start are masked per lane;
//     waves whose tokens have no sequence start among their taps skip it.
#include "lowrank_common.h"

namespace dsc {
namespace {

constexpr int kDzWaves = 4;  // waves per block, one token range each
constexpr int kDzBlock = kDzWaves * kWave;

struct DzParams {
    const uint16_t *x, *g;  // (N, D)
    const uint16_t *Ut;     // (W, R, D): U with the tap outermost
    float *parts;           // (S, N, R) fp32: one region per channel split
    SeqMap seq;
    int64_t N, D;
    int32_t R;
    int64_t ntb;   // token blocks
    int64_t cper;  // channels per split, a multiple of 32
    int32_t S;
};

template <int W, int RT>
struct DzLds {
    static constexpr int RP = 16 * RT;  // ranks padded to whole tiles
    static constexpr int kPitch = 80;   // bytes per (tap, rank) row: 32 channels + 16 B against bank conflicts
    static constexpr int kBuf = W * RP * kPitch;
    static constexpr int kPieces = W * RP * 4;  // 16-byte pieces of one slice
    static constexpr int kPerThread = (kPieces + kDzBlock - 1) / kDzBlock;
};

template <int W, int RT, int MT>
__global__ __launch_bounds__(kDzBlock, 2) void lr_dz_kernel(DzParams p) {
    using L = DzLds<W, RT>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * L::kBuf];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t split = blockIdx.x / p.ntb;
    const int64_t tb = blockIdx.x - split * p.ntb;
    const int64_t n0 = (tb * kDzWaves + wid) * 16 * MT;  // the wave's first token
    const int64_t cs = split * p.cper;
    const int64_t ce = min(cs + p.cper, p.D);
    const int nch = (int)((ce - cs + 31) / 32);
    const int tok = lane & 15, q = lane >> 4;
    const int64_t N = p.N, D = p.D;
    const int R = p.R;

    // taps k <= back[mt] of the lane's token stay inside its sequence
    int back[MT];
    bool masked = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t n = n0 + 16 * mt + tok;
        back[mt] = W - 1;
        if (n < N) {
            int64_t s, e;
            p.seq.find(n, s, e);
            back[mt] = (int)min((int64_t)(W - 1), n - s);
        }
        masked = masked || back[mt] < W - 1;
    }
    masked = __builtin_amdgcn_ballot_w64(masked) != 0;  // wave-uniform

    // U slice staging: piece i of a slice = 16 bytes (8 channels) of row (tap k, rank r).
    // Every load is issued, at an address clamped into the tensor, and pieces
    // outside R or the split are zeroed afterwards: branch-free loads keep the
    // compiler's count of loads in flight exact, so the prefetch overlaps.
    uint4 ustage[L::kPerThread];
    auto fetch_u = [&](int64_t c0) {
#pragma unroll
        for (int j = 0; j < L::kPerThread; ++j) {
            const int piece = (int)threadIdx.x + j * kDzBlock;
            const int row = piece >> 2, part = piece & 3;
            const int k = min(row / L::RP, W - 1), r = row - (row / L::RP) * L::RP;
            const int64_t ch = c0 + 8 * part;
            const bool ok = piece < L::kPieces && r < R && ch < ce;
            const int64_t off = ((int64_t)k * R + min(r, R - 1)) * D + min(ch, D - 8);
            const uint4 v = ld_u4<false>(p.Ut + off);
            ustage[j] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_u = [&](int buf) {
#pragma unroll
        for (int j = 0; j < L::kPerThread; ++j) {
            const int piece = (int)threadIdx.x + j * kDzBlock;
            if (piece < L::kPieces)
                *reinterpret_cast<uint4 *>(lds + buf * L::kBuf + (piece >> 2) * L::kPitch + 16 * (piece & 3)) =
                    ustage[j];
        }
    };

    // dy and x of the wave's tokens for 32 channels (8 per lane), branch-free
    // as above: rows past N and channels past the split read a clamped
    // address and are zeroed
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    auto fetch_act = [&](int64_t c0, uint4 (&xr)[MT], uint4 (&gr)[MT], uint4 &xh) {
        const int64_t ch = c0 + 8 * q;
        const bool ok = ch < ce;  // D % 8 == 0: a lane's 8 channels are all in or all out
        const int64_t chc = min(ch, D - 8);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t n = n0 + 16 * mt + tok;
            const int64_t off = min(n, N - 1) * D + chc;
            const uint4 xv = ld_u4<true>(p.x + off);
            const uint4 gv = ld_u4<true>(p.g + off);
            const bool in = ok && n < N;
            xr[mt] = in ? xv : zero4;
            gr[mt] = in ? gv : zero4;
        }
        // the W-1 rows before the wave's first token (the taps of its first tile)
        const int64_t nh = n0 - 16 + tok;
        const uint4 hv = ld_u4<false>(p.x + min(max(nh, (int64_t)0), N - 1) * D + chc);
        xh = (W > 1 && ok && tok >= 16 - (W - 1) && nh >= 0 && nh < N) ? hv : zero4;
    };

    floatx4 acc[MT][RT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[mt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};

    uint4 xr[MT], gr[MT], xh;
    fetch_u(cs);
    store_u(0);
    fetch_act(cs, xr, gr, xh);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        const int64_t cn = cs + 32 * (int64_t)(c + 1);
        const bool more = c + 1 < nch;  // block-uniform
        // the next 32 channels (past the split's end on the last chunk: loads of
        // clamped addresses whose values are zeroed and never used)
        uint4 nxr[MT], ngr[MT], nxh;
        fetch_u(cn);
        fetch_act(cn, nxr, ngr, nxh);
        // keep these loads ahead of the products below (left to itself the
        // scheduler sinks them to the end of the iteration, where nothing
        // overlaps their latency)
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char *us = lds + buf * L::kBuf;
#pragma unroll
        for (int k = 0; k < W; ++k) {
            bf16x8 ua[RT];  // A: rows = ranks 16rt + (lane&15), K = channels 8q..8q+7 of the slice
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                ua[rt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const uint4 *>(us + (k * L::RP + 16 * rt + tok) * L::kPitch + 16 * q));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t xc[4] = {xr[mt].x, xr[mt].y, xr[mt].z, xr[mt].w};
                const uint4 pv = mt == 0 ? xh : xr[mt > 0 ? mt - 1 : 0];
                const uint32_t xp[4] = {pv.x, pv.y, pv.z, pv.w};
                uint32_t xk[4];
                if (k == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xk[i] = xc[i];
                } else {
                    shift_back4<W>(k, xc, xp, xk);
                }
                if (masked) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xk[i] = k <= back[mt] ? xk[i] : 0u;
                }
                const uint32_t gc[4] = {gr[mt].x, gr[mt].y, gr[mt].z, gr[mt].w};
                uint32_t dw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dw[i] = pack_bf16x2(bf16_lo(gc[i]) * bf16_lo(xk[i]), bf16_hi(gc[i]) * bf16_hi(xk[i]));
                const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(dw[0], dw[1], dw[2], dw[3]));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[mt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[rt], b, acc[mt][rt], 0, 0, 0);
            }
        }
        if (more) {
            store_u(buf ^ 1);  // the other buffer: its last readers finished before the previous barrier
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                xr[mt] = nxr[mt];
                gr[mt] = ngr[mt];
            }
            xh = nxh;
        }
        __syncthreads();
    }

    // partial dz of this split: acc[mt][rt][j] = dz(token n0 + 16mt + tok, rank 16rt + 4q + j)
    float *dst = p.parts + split * N * R;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t n = n0 + 16 * mt + tok;
        if (n >= N) continue;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * q + j;
                if (r < R) dst[n * R + r] = acc[mt][rt][j];
            }
    }
}

// Ut[(k*R + r)*D + d] = U[(r*D + d)*W + k]: the tap-major copy of U.
template <int W>
__global__ __launch_bounds__(256) void transpose_u_kernel(const uint16_t *U, uint16_t *Ut, int64_t R, int64_t D) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (r, d)
    if (i >= R * D) return;
    const int64_t r = i / D, d = i - r * D;
    uint16_t v[W];
    load_taps<W>(U + i * W, v);
#pragma unroll
    for (int k = 0; k < W; ++k) Ut[((int64_t)k * R + r) * D + d] = v[k];
}

template <int W, int RT, int MT>
hipError_t launch_dz(const DzParams &p, hipStream_t st) {
    const int64_t blocks = p.ntb * p.S;
    if (blocks) hipLaunchKernelGGL((lr_dz_kernel<W, RT, MT>), dim3((unsigned)blocks), dim3(kDzBlock), 0, st, p);
    return hipGetLastError();
}

template <int W>
hipError_t dz_rt(const DzParams &p, hipStream_t st) {
    switch ((p.R + 15) / 16) {
        case 1: return launch_dz<W, 1, 4>(p, st);
        case 2: return launch_dz<W, 2, 4>(p, st);
        case 3: return launch_dz<W, 3, 4>(p, st);
        case 4: return launch_dz<W, 4, 4>(p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

LrDzPlan lowrank_dz_plan(int64_t N, int64_t D, int32_t W, int32_t R) {
    LrDzPlan pl;
    constexpr int MT = 4;
    pl.ntb = (N + kDzWaves * 16 * MT - 1) / (kDzWaves * 16 * MT);
    // about 2048 waves (two per SIMD on a 256-CU device), in whole 32-channel slices;
    // the split depends on the sizes only, so the order of summation does too
    const int64_t slices = (D + 31) / 32;
    int64_t S = (512 + pl.ntb - 1) / (pl.ntb > 0 ? pl.ntb : 1);
    S = S < 1 ? 1 : (S > slices ? slices : S);
    pl.cper = ((slices + S - 1) / S) * 32;
    pl.S = (int32_t)((D + pl.cper - 1) / pl.cper);
    pl.ut_elems = (int64_t)W * R * D;
    pl.part_floats = (int64_t)pl.S * N * R;
    (void)W;
    return pl;
}

bool lowrank_dz_supported(int32_t W, int32_t R) { return W >= 1 && W <= 8 && R >= 1 && R <= 64; }

hipError_t lowrank_dz_partials(const LrProblem &pr, const LrDzPlan &pl, uint16_t *Ut, float *parts, hipStream_t st) {
    const int64_t RD = (int64_t)pr.R * pr.D;
    if (RD == 0 || pr.N == 0) return hipSuccess;
    const uint16_t *U = static_cast<const uint16_t *>(pr.U);
    const dim3 tg((unsigned)((RD + 255) / 256));
    switch (pr.W) {
        case 1: hipLaunchKernelGGL(transpose_u_kernel<1>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 2: hipLaunchKernelGGL(transpose_u_kernel<2>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 3: hipLaunchKernelGGL(transpose_u_kernel<3>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 4: hipLaunchKernelGGL(transpose_u_kernel<4>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 5: hipLaunchKernelGGL(transpose_u_kernel<5>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 6: hipLaunchKernelGGL(transpose_u_kernel<6>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 7: hipLaunchKernelGGL(transpose_u_kernel<7>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        case 8: hipLaunchKernelGGL(transpose_u_kernel<8>, tg, dim3(256), 0, st, U, Ut, (int64_t)pr.R, pr.D); break;
        default: return hipErrorInvalidValue;
    }
    DzParams p;
    p.x = static_cast<const uint16_t *>(pr.x);
    p.g = static_cast<const uint16_t *>(pr.dy);
    p.Ut = Ut;
    p.parts = parts;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N;
    p.D = pr.D;
    p.R = pr.R;
    p.ntb = pl.ntb;
    p.cper = pl.cper;
    p.S = pl.S;
    switch (pr.W) {
        case 1: return dz_rt<1>(p, st);
        case 2: return dz_rt<2>(p, st);
        case 3: return dz_rt<3>(p, st);
        case 4: return dz_rt<4>(p, st);
        case 5: return dz_rt<5>(p, st);
        case 6: return dz_rt<6>(p, st);
        case 7: return dz_rt<7>(p, st);
        case 8: return dz_rt<8>(p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsc
