// lowrank_fwd.hip -- wide low-rank forward for gfx950 (R <= 64, bf16).
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: parametrization (1) low-rank factorisation;
// Efficient training implementation: z and U are read, zU is formed on chip
// and the convolution follows at once):
//   w[n,d,k] = sum_{r<R} z[n,r] * U[r, d*W+k]
//   y[n,d]   = rho*x[n,d] + sum_{k<W, n-k in seq(n)} w[n,d,k] * x[n-k,d]
//
// Built on its own so that its matrix-core results can live in ordinary
// vector registers (the build passes -amdgpu-mfma-vgpr-form for this file
// only; the backward kernels keep the default register form).
#include "lowrank_common.h"

namespace dsc {
namespace {

// Wide forward for R <= 32: a wave owns 64 channels (two 32-channel slices,
// one 128-byte line of every token row) and walks a token range in 16-token
// steps.  x and y move as 8 token rows x 128 bytes per wave instruction
// (lane = row rl, chunk cl), whole cache lines, and pass through a per-wave
// LDS tile to and from the matrix-core layout (lane = token, chunk q of each
// slice).  The causal taps read x rows tok-k straight from the LDS ring, so
// no lane shifts are needed; z rows (the B operand) are loaded once per step
// for both slices.
struct FwdWideLds {
    static constexpr int kRow = 128;        // bytes per token row: 64 bf16 channels
    static constexpr int kX = 40 * kRow;    // 8 mirror rows + two 16-row slots
    static constexpr int kY = 16 * kRow;    // y tile of one step
    static constexpr int kWave = kX + kY;
};

// Byte offset of 16-byte chunk c (0..7) of physical LDS row r.  The chunk sits
// at position c ^ ((r >> 1) & 7), so 16 consecutive rows read at one chunk
// and 8 chunks of one row both spread over distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * FwdWideLds::kRow + 16 * (c ^ ((r >> 1) & 7)); }

// ROPE: the output's channels below p.rot are then turned pair by pair at
// the token's position in its sequence ("RoFormer: Enhanced Transformer with
// Rotary Position Embedding", Su et al., Section 3.4.2), on the fp32 result
// before it is rounded.
template <int W, int RC, int PF, bool RVEC, bool ROPE = false>
__global__ __launch_bounds__(kBlock) void lr_fwd_wide(LrParams p, int64_t npairs, int64_t tok_per_wave) {
    using L = FwdWideLds;
    static_assert(PF % 2 == 0, "x ring slots alternate with the step parity");
    static_assert(W <= 8, "the LDS ring mirrors 7 rows of the previous step");
    __shared__ __attribute__((aligned(16))) unsigned char lds[(kBlock / kWave) * L::kWave];
    __shared__ uint32_t seq_words[kBlock / kWave][kSeqWords];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = (int64_t)blockIdx.x * (kBlock / kWave) + wid;
    const int64_t tchunk = wave / npairs;
    const int64_t pair = wave - tchunk * npairs;
    const int64_t nbeg = tchunk * tok_per_wave;
    if (nbeg >= p.N) return;  // wave-uniform; the kernel has no block barrier
    const int64_t nend = min(nbeg + tok_per_wave, p.N);
    const int nsteps = (int)((nend - nbeg + 15) / 16);

    const int64_t D = p.D;
    const int R = p.R;
    const int64_t c0 = pair * 64;  // first channel of the wave
    const int tok = lane & 15, q = lane >> 4;  // matrix-core layout
    const int rl = lane >> 3, cl = lane & 7;   // row layout

    const uint16_t *U = static_cast<const uint16_t *>(p.U);
    const uint16_t *xg = static_cast<const uint16_t *>(p.x);
    const uint16_t *zg = static_cast<const uint16_t *>(p.z);
    uint16_t *yg = static_cast<uint16_t *>(p.y);

    bf16x8 ua[2][W][2][RC];  // per slice: U_k^T rows (channels) x K (rank)
    load_u_rows<W, RC>(U, R, D, c0, lane, ua[0]);
    load_u_rows<W, RC>(U, R, D, c0 + 32, lane, ua[1]);

    // streams over the wave's rows [nbeg, nend)
    const uint32_t act_step = (uint32_t)(16 * D * 2);
    const uint32_t half_step = (uint32_t)(8 * D * 2);
    const uint32_t z_step = (uint32_t)(16 * R * 2);
    const bool row_ok = c0 + 8 * cl < D;  // D % 8 == 0: a chunk is all in or out
    const uint32_t roff = row_ok ? (uint32_t)((rl * D + c0 + 8 * cl) * 2) : kFar;
    uint32_t zoff[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        const int r0 = 32 * c + 8 * q;
        zoff[c] = r0 < R ? (uint32_t)((tok * R + r0) * 2) : kFar;
    }
    const __amdgpu_buffer_rsrc_t rx = make_stream(xg + nbeg * D, (nend - nbeg) * D * 2);
    const __amdgpu_buffer_rsrc_t rz = make_stream(zg + nbeg * R, (nend - nbeg) * R * 2);
    const __amdgpu_buffer_rsrc_t ry = make_stream(yg + nbeg * D, (nend - nbeg) * D * 2);

    auto fetch_x = [&](int step, uint4 (&xd)[2]) {
        xd[0] = buf_load16<kLrNtX>(rx, roff + (uint32_t)step * act_step);
        xd[1] = buf_load16<kLrNtX>(rx, roff + half_step + (uint32_t)step * act_step);
    };
    auto fetch_z = [&](int step, uint4 (&zd)[RC]) {
        if constexpr (RVEC) {
#pragma unroll
            for (int c = 0; c < RC; ++c) zd[c] = buf_load16(rz, zoff[c] + (uint32_t)step * z_step);
        } else {
            const int64_t n = nbeg + 16 * (int64_t)step + tok;
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
    };

    unsigned char *xl = lds + wid * L::kWave;  // [8 mirror rows][slot 0: 16 rows][slot 1: 16 rows]
    unsigned char *yl = xl + L::kX;            // [16 rows]
    // x rows of a step into ring slot `slot` (= step parity); slot 1 also
    // copies its tokens 9..15 to the mirror rows 1..7, which slot 0 reads as
    // the previous step's tail
    auto put_x = [&](int slot, const uint4 (&v)[2]) {
        const int b = 8 + 16 * slot;
        *reinterpret_cast<uint4 *>(xl + swz(b + rl, cl)) = v[0];
        *reinterpret_cast<uint4 *>(xl + swz(b + 8 + rl, cl)) = v[1];
        if (slot == 1 && rl >= 1) *reinterpret_cast<uint4 *>(xl + swz(rl, cl)) = v[1];
    };

    StartBits<kSeqWords> starts;
    starts.build(seq_words[wid], p.seq, p.N, nbeg - 32, lane);
    SeqPos sp{0};
    RopeCarry rc[ROPE ? 2 : 1];   // the lane's two 8-channel chunks (one per slice)
    float r16[ROPE ? 2 : 1][8];   // their turn by 16 positions (table row 16)
    if constexpr (ROPE) {
        int64_t s_, e_;
        p.seq.find(nbeg < p.N ? nbeg : p.N - 1, s_, e_);
        sp.start = s_;
    }

    // the previous step's tail (tokens nbeg-7 .. nbeg-1) into slot 1 and the mirror
    {
        uint4 v[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
        const int64_t n = nbeg - 8 + rl;
        if (n >= 0 && row_ok) v[1] = *reinterpret_cast<const uint4 *>(xg + n * D + c0 + 8 * cl);
        put_x(1, v);
    }

    uint4 xq[PF][2];
    uint4 zq[PF][RC];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        fetch_x(i, xq[i]);
        fetch_z(i, zq[i]);
    }

    for (int s0 = 0; s0 < nsteps; s0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int s = s0 + i;
            const int slot = i & 1;  // s0 is a multiple of PF (even)
            const int base = 8 + 16 * slot;
            wave_lds_fence();  // the previous step's LDS reads come before these writes
            put_x(slot, xq[i]);
            fetch_x(s + PF, xq[i]);
            wave_lds_fence();  // other lanes read these rows below

            // sequence starts among the step's reach (bit j of win <-> token nbeg+16s-(W-1)+j);
            // taps k > nv of a token reach before its sequence
            uint32_t win = 0;
            if constexpr (W > 1) win = __builtin_amdgcn_readfirstlane(starts.window(nbeg + 16 * (int64_t)s - (W - 1)));
            const bool masked = (win & (((1u << (W + 14)) - 1u) << 1)) != 0u;  // wave-uniform
            if constexpr (ROPE) {
                const int64_t pos = sp.pos_and_advance(starts, nbeg + 16 * (int64_t)s, tok);
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    if (s == 0) {
                        rc[sl].start(p, pos, c0 + 32 * sl + 8 * q);
                        rope_cs<8>(p, 16, c0 + 32 * sl + 8 * q, r16[sl]);
                    } else {
                        rc[sl].advance(p, pos, c0 + 32 * sl + 8 * q, r16[sl],
                                       rope_restart(starts, nbeg + 16 * (int64_t)s));
                    }
                }
            }

#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                uint32_t xs[W][4];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(xl + swz(base + tok - k, q + 4 * sl));
                    xs[k][0] = v.x; xs[k][1] = v.y; xs[k][2] = v.z; xs[k][3] = v.w;
                }
                if constexpr (W > 1) {
                    if (masked) {
                        const uint32_t sub = (win >> (tok + 1)) & ((1u << (W - 1)) - 1u);
                        const int nv = sub ? (W - 2) - (31 - __builtin_clz(sub)) : W - 1;
#pragma unroll
                        for (int k = 1; k < W; ++k)
                            if (k > nv)
#pragma unroll
                                for (int e = 0; e < 4; ++e) xs[k][e] = 0u;
                    }
                }
                floatx4 acc[W][2];
#pragma unroll
                for (int k = 0; k < W; ++k)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            ua[sl][k][t][0], __builtin_bit_cast(bf16x8, zq[i][0]), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                        for (int c = 1; c < RC; ++c)
                            acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                ua[sl][k][t][c], __builtin_bit_cast(bf16x8, zq[i][c]), acc[k][t], 0, 0, 0);
                    }
                float out[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int t = c >> 2, j = c & 3;
                    const uint32_t x0 = xs[0][c >> 1];
                    float a = __uint_as_float(((c & 1) ? (x0 & 0xffff0000u) : (x0 << 16)) & p.rmask);
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const uint32_t v = xs[k][c >> 1];
                        a = __builtin_fmaf(acc[k][t][j], (c & 1) ? bf16_hi(v) : bf16_lo(v), a);
                    }
                    out[c] = a;
                }
                if constexpr (ROPE) {
                    // the lane's 8 channels: 4 pairs of one head
                    if (c0 + 32 * sl + 8 * q < p.rot) turn<8, false>(out, rc[sl].c);
                }
                uint4 yv;
                yv.x = pack_bf16x2(out[0], out[1]);
                yv.y = pack_bf16x2(out[2], out[3]);
                yv.z = pack_bf16x2(out[4], out[5]);
                yv.w = pack_bf16x2(out[6], out[7]);
                *reinterpret_cast<uint4 *>(yl + swz(tok, q + 4 * sl)) = yv;
            }
            fetch_z(s + PF, zq[i]);
            wave_lds_fence();  // the y tile written above is read in row layout by other lanes
            {
                const uint4 y0 = *reinterpret_cast<const uint4 *>(yl + swz(rl, cl));
                const uint4 y1 = *reinterpret_cast<const uint4 *>(yl + swz(8 + rl, cl));
                buf_store16<kLrNtY>(ry, roff + (uint32_t)s * act_step, y0);
                buf_store16<kLrNtY>(ry, roff + half_step + (uint32_t)s * act_step, y1);
            }
        }
    }
}

#ifndef DSC_LR_FWD_WIDE_PF1
#define DSC_LR_FWD_WIDE_PF1 4
#endif
#ifndef DSC_LR_FWD_WIDE_PF2
#define DSC_LR_FWD_WIDE_PF2 2
#endif
// Prefetch depth in steps (measured on MI355X).  At R > 32 a depth of 2 keeps
// the kernel within 256 VGPRs, i.e. 2 waves per SIMD.
template <int RC>
constexpr int wide_pf() { return RC == 1 ? DSC_LR_FWD_WIDE_PF1 : DSC_LR_FWD_WIDE_PF2; }

template <int W, int RC, bool ROPE>
hipError_t mfma_fwd_wide(const LrProblem &pr, hipStream_t st) {
    constexpr int PF = wide_pf<RC>();
    LrParams p = make_params<BF16>(pr);
    const int64_t npairs = (p.D + 63) / 64;
    const int64_t cap = walk_cap(p.D, 16 * PF, 16 * (2 * PF + 2));
    if (cap < 16 * PF) return hipErrorNotSupported;  // the caller falls back
    static const int bpc_vec =
        blocks_per_cu(reinterpret_cast<const void *>(&lr_fwd_wide<W, RC, PF, true, ROPE>), kBlock);
    static const int bpc_gather =
        blocks_per_cu(reinterpret_cast<const void *>(&lr_fwd_wide<W, RC, PF, false, ROPE>), kBlock);
    const bool rvec = p.R % 8 == 0;
    const int64_t slots = (int64_t)device_cus() * (rvec ? bpc_vec : bpc_gather) * (kBlock / kWave);
    const int64_t tpw = walk_length(p.N, npairs, slots, cap, 16 * PF, kWaveFixedTokens);
    const int64_t waves = ((p.N + tpw - 1) / tpw) * npairs;
    const int64_t b = (waves + 3) / 4;
    if (b) {
        if (rvec)
            hipLaunchKernelGGL((lr_fwd_wide<W, RC, PF, true, ROPE>), dim3((unsigned)b), dim3(kBlock), 0, st, p, npairs,
                               tpw);
        else
            hipLaunchKernelGGL((lr_fwd_wide<W, RC, PF, false, ROPE>), dim3((unsigned)b), dim3(kBlock), 0, st, p,
                               npairs, tpw);
    }
    return hipGetLastError();
}

template <int W>
hipError_t wide_rc(const LrProblem &pr, hipStream_t st, bool *used) {
    hipError_t e = hipErrorNotSupported;
    const bool rope = pr.rot > 0;
    switch ((pr.R + 31) / 32) {
        case 1: e = rope ? mfma_fwd_wide<W, 1, true>(pr, st) : mfma_fwd_wide<W, 1, false>(pr, st); break;
        case 2: e = rope ? mfma_fwd_wide<W, 2, true>(pr, st) : mfma_fwd_wide<W, 2, false>(pr, st); break;
        default: break;
    }
    *used = e != hipErrorNotSupported;
    return e;
}

}  // namespace

hipError_t lowrank_fwd_wide(const LrProblem &p, hipStream_t s, bool *used) {
    *used = false;
    if (p.dtype != Dtype::BF16) return hipErrorNotSupported;
    switch (p.W) {
        case 1: return wide_rc<1>(p, s, used);
        case 2: return wide_rc<2>(p, s, used);
        case 3: return wide_rc<3>(p, s, used);
        case 4: return wide_rc<4>(p, s, used);
        case 5: return wide_rc<5>(p, s, used);
        case 6: return wide_rc<6>(p, s, used);
        case 7: return wide_rc<7>(p, s, used);
        case 8: return wide_rc<8>(p, s, used);
        default: return hipErrorNotSupported;
    }
}

}  // namespace dsc
