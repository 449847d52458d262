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
// bf16 forward: the R-wide contraction runs on the matrix cores
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
    int64_t nchunks;
};

constexpr int kBlock = 256;

// ---------------------------------------------------------------- generic

// One thread per (token, 16-byte channel chunk).
template <class E, int W>
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
    Vec16<E>::store(static_cast<S *>(p.y) + n * p.D + d0, acc);
}

template <class E, int W>
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

    // dx: filters of the W tokens m..m+W-1 that read x[m]
    float gm[VEC], acc[VEC];
    Vec16<E>::load(g + m * p.D + d0, gm);
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
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[c] = __builtin_fmaf(wk[c], gt[c], acc[c]);
        }
    }
    Vec16<E>::store(static_cast<S *>(p.dx) + m * p.D + d0, acc);

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

// DPP controls (row = 16 lanes): lane i of a row reads lane i-k (shr) or
// lane (i-k) mod 16 (ror).
template <int K>
__device__ __forceinline__ uint32_t shift_in_row(uint32_t cur, uint32_t prev) {
    const int rot = __builtin_amdgcn_mov_dpp((int)prev, 0x120 + K, 0xf, 0xf, true);
    return (uint32_t)__builtin_amdgcn_update_dpp(rot, (int)cur, 0x110 + K, 0xf, 0xf, false);
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
template <int W, int RC, int PF>
__global__ __launch_bounds__(kBlock) void lr_fwd_mfma(LrParams p, int64_t nslices, int64_t tok_per_wave) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    const int64_t tchunk = wave / nslices;
    const int64_t slice = wave - tchunk * nslices;
    const int64_t d0 = slice * 32;
    const int64_t nbeg = tchunk * tok_per_wave;
    if (nbeg >= p.N) return;  // wave-uniform
    const int64_t nend = min(nbeg + tok_per_wave, p.N);
    const int64_t nsteps = (nend - nbeg + 15) / 16;

    const int tok = lane & 15;
    const int q = lane >> 4;
    const int64_t cbase = d0 + 8 * q;
    const bool chan_ok = cbase < p.D;  // D % 8 == 0: a lane's 8 channels are all in or out
    const int R = p.R;
    const int64_t DW = p.D * W;

    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    const uint16_t *z = static_cast<const uint16_t *>(p.z);
    const uint16_t *U = static_cast<const uint16_t *>(p.U);
    uint16_t *y = static_cast<uint16_t *>(p.y);

    // A operands: U_k^T rows (channels) x K (rank), per tap k, tile t, K chunk c.
    bf16x8 ua[W][2][RC];
    {
        const int row = lane & 15;
        const int kq = lane >> 4;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t ch = d0 + 8 * (row >> 2) + 4 * t + (row & 3);
#pragma unroll
            for (int c = 0; c < RC; ++c) {
#pragma unroll
                for (int k = 0; k < W; ++k) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = 32 * c + 8 * kq + i;
                        uint16_t v = 0;
                        if (r < R && ch < p.D) v = U[(int64_t)r * DW + ch * W + k];
                        ua[k][t][c][i] = __builtin_bit_cast(__bf16, v);
                    }
                }
            }
        }
    }

    auto load_x = [&](int64_t n, uint32_t (&dst)[4]) {
        if (n < nend && chan_ok) {
            uint4 v = *reinterpret_cast<const uint4 *>(x + n * p.D + cbase);
            dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
        } else {
            dst[0] = dst[1] = dst[2] = dst[3] = 0u;
        }
    };
    // B operand: Z^T, K = rank 32c + 8q .. +7, column = token
    const bool r_vec = (R % 8) == 0;
    auto load_z = [&](int64_t n, bf16x8 (&dst)[RC]) {
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            const int r0 = 32 * c + 8 * q;
            if (n < nend && r0 < R) {
                if (r_vec) {
                    dst[c] = *reinterpret_cast<const bf16x8 *>(z + n * R + r0);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint16_t v = (r0 + i < R) ? z[n * R + r0 + i] : (uint16_t)0;
                        dst[c][i] = __builtin_bit_cast(__bf16, v);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) dst[c][i] = __builtin_bit_cast(__bf16, (uint16_t)0);
            }
        }
    };

    // previous step's x for the taps that reach back across the step edge
    uint32_t xprev[4];
    {
        const int64_t n = nbeg - 16 + tok;
        if (n >= 0 && tok >= 16 - (W - 1) && chan_ok) {
            uint4 v = *reinterpret_cast<const uint4 *>(x + n * p.D + cbase);
            xprev[0] = v.x; xprev[1] = v.y; xprev[2] = v.z; xprev[3] = v.w;
        } else {
            xprev[0] = xprev[1] = xprev[2] = xprev[3] = 0u;
        }
    }

    uint32_t xq[PF][4];
    bf16x8 zq[PF][RC];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        load_x(nbeg + 16 * i + tok, xq[i]);
        load_z(nbeg + 16 * i + tok, zq[i]);
    }

    for (int64_t st = 0; st < nsteps; st += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (st + i < nsteps) {
                const int64_t nstep = nbeg + 16 * (st + i);
                const int64_t n = nstep + tok;
                uint32_t xc[4] = {xq[i][0], xq[i][1], xq[i][2], xq[i][3]};
                bf16x8 zc[RC];
#pragma unroll
                for (int c = 0; c < RC; ++c) zc[c] = zq[i][c];
                if (st + i + PF < nsteps) {
                    load_x(n + 16 * PF, xq[i]);
                    load_z(n + 16 * PF, zq[i]);
                }

                floatx4 acc[W][2];
#pragma unroll
                for (int k = 0; k < W; ++k)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        acc[k][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < RC; ++c)
                            acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[k][t][c], zc[c], acc[k][t], 0, 0, 0);
                    }

                Shifted<W> xs;
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) xs.v[0][i2] = xc[i2];
                fill_shift<W, 1>(xs, xc, xprev);

                // sequence masking: only when a boundary can touch this step
                int64_t s0, e0;
                p.seq.find(nstep, s0, e0);
                const bool clean = (e0 >= nstep + 16) && (nstep - s0 >= W - 1);
                if (!clean) {
                    int64_t s, e;
                    p.seq.find(n < p.N ? n : p.N - 1, s, e);
                    const int64_t nv = n - s;
#pragma unroll
                    for (int k = 1; k < W; ++k)
                        if (k > nv)
#pragma unroll
                            for (int i2 = 0; i2 < 4; ++i2) xs.v[k][i2] = 0u;
                }

                float out[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int t = c >> 2, j = c & 3;
                    float a = p.rho * ((c & 1) ? bf16_hi(xc[c >> 1]) : bf16_lo(xc[c >> 1]));
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const uint32_t v = xs.v[k][c >> 1];
                        const float xk = (c & 1) ? bf16_hi(v) : bf16_lo(v);
                        a = __builtin_fmaf(acc[k][t][j], xk, a);
                    }
                    out[c] = a;
                }
                if (n < nend && chan_ok) {
                    uint4 v;
                    v.x = pack_bf16x2(out[0], out[1]);
                    v.y = pack_bf16x2(out[2], out[3]);
                    v.z = pack_bf16x2(out[4], out[5]);
                    v.w = pack_bf16x2(out[6], out[7]);
                    *reinterpret_cast<uint4 *>(y + n * p.D + cbase) = v;
                }
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) xprev[i2] = xc[i2];
            }
        }
    }
}

// ------------------------------------------------------------ small kernels

__global__ void fill_zero_f32(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

__global__ void cast_f32_bf16(const float *src, uint16_t *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) dst[i] = to_bf16(src[i]);
}

int64_t nblocks(int64_t n) { return (n + kBlock - 1) / kBlock; }

template <class E>
LrParams make_params(const LrProblem &pr) {
    LrParams p;
    p.x = pr.x; p.z = pr.z; p.U = pr.U; p.dy = pr.dy;
    p.y = pr.y; p.dx = pr.dx; p.dz = pr.dz;
    p.dU = pr.dU; p.dzacc = pr.dz_acc;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N; p.D = pr.D; p.R = pr.R;
    p.rho = pr.residual ? 1.f : 0.f;
    p.nchunks = pr.D / E::kVec;
    return p;
}

template <class E, int W>
hipError_t generic_fwd(const LrProblem &pr, hipStream_t st) {
    LrParams p = make_params<E>(pr);
    const int64_t b = nblocks(p.N * p.nchunks);
    if (b) hipLaunchKernelGGL((lr_fwd_generic<E, W>), dim3((unsigned)b), dim3(kBlock), 0, st, p);
    return hipGetLastError();
}

template <class E, int W>
hipError_t generic_bwd(const LrProblem &pr, hipStream_t st) {
    LrParams p = make_params<E>(pr);
    const int64_t nU = (int64_t)p.R * p.D * W;
    const int64_t nz = p.N * p.R;
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)nblocks(nU)), dim3(kBlock), 0, st, p.dU, nU);
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, p.dzacc, nz);
    const int64_t b = nblocks(p.N * p.nchunks);
    if (b) hipLaunchKernelGGL((lr_bwd_generic<E, W>), dim3((unsigned)b), dim3(kBlock), 0, st, p);
    if constexpr (sizeof(typename E::store_t) == 2)
        hipLaunchKernelGGL(cast_f32_bf16, dim3((unsigned)nblocks(nz)), dim3(kBlock), 0, st, p.dzacc,
                           static_cast<uint16_t *>(p.dz), nz);
    return hipGetLastError();
}

constexpr int kPF = 4;
constexpr int64_t kTargetWaves = 256 * 8;

template <int W, int RC>
hipError_t mfma_fwd(const LrProblem &pr, hipStream_t st) {
    LrParams p = make_params<BF16>(pr);
    const int64_t nslices = (p.D + 31) / 32;
    int64_t tpw = (p.N * nslices + kTargetWaves - 1) / kTargetWaves;
    tpw = ((tpw + 15) / 16) * 16;
    if (tpw < 16 * kPF) tpw = 16 * kPF;
    const int64_t nchunks_t = (p.N + tpw - 1) / tpw;
    const int64_t waves = nchunks_t * nslices;
    const int64_t b = (waves + 3) / 4;
    if (b) hipLaunchKernelGGL((lr_fwd_mfma<W, RC, kPF>), dim3((unsigned)b), dim3(kBlock), 0, st, p, nslices, tpw);
    return hipGetLastError();
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

size_t lowrank_bwd_workspace(Dtype dt, int64_t N, int64_t D, int32_t W, int32_t R) {
    (void)D; (void)W;
    if (dt == Dtype::F32) return 0;
    const size_t bytes = (size_t)N * (size_t)R * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t lowrank_fwd(const LrProblem &p, hipStream_t s) {
    if (p.dtype == Dtype::BF16) {
        DSC_W_SWITCH(p.W, mfma_fwd_rc<Wc>(p, s));
    }
    DSC_W_SWITCH(p.W, (generic_fwd<F32, Wc>(p, s)));
}

hipError_t lowrank_bwd(const LrProblem &p, hipStream_t s) {
    if (p.dtype == Dtype::BF16) {
        DSC_W_SWITCH(p.W, (generic_bwd<BF16, Wc>(p, s)));
    }
    DSC_W_SWITCH(p.W, (generic_bwd<F32, Wc>(p, s)));
}

}  // namespace dsc
