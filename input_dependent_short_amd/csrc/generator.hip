// generator.hip -- head-wise dynamic short convolution whose filters are
// generated from the hidden state on chip, for gfx950 ("Dynamic Short
// Convolutions Improve Transformers", gist.science technical summary,
// Methodology: parametrization -- the filter of token t is a learned linear
// map of the current hidden state; head-wise tying over H channels).
//
//   w[n, g*W + k] = sum_{j<K} h[n, j] * V[g*W + k, j]            (on chip only)
//   y[n, d]       = rho*x[n,d] + sum_{k<W, n-k in seq(n)} w[n, (d/H)*W + k] * x[n-k, d]
// Backward for L = <dy, y>:
//   dx[m, d]      = rho*dy[m,d] + sum_{k<W, m+k in seq(m)} w[m+k, (d/H)*W + k] * dy[m+k, d]
//   dw[n, g*W+k]  = sum_{d in group g, n-k in seq(n)} dy[n,d] * x[n-k,d]
//   dh = dw V,  dV = dw^T h
//
// The map is a GEMM (N x K) . (K x G*W) on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  A block computes a tile of
// 128 tokens x TG groups * W taps of w, parks it in LDS and runs the
// convolution of those tokens over the TG groups' channels as its epilogue:
// w never reaches HBM.  The backward recomputes w the same way, with tiles
// that overlap by W-1 tokens (dx of token m reads the filters of m..m+W-1),
// forms dx and the filter gradient dw of the tile's tokens in the epilogue,
// and writes dw once (bf16) for the two products dh = dw V and dV = dw^T h,
// which the same GEMM core runs with plain epilogues.
#include "dsc_common.h"
#include "dsc_kernels.h"

namespace dsc {
namespace {

constexpr int kGBlock = 256;   // 4 waves; wave v owns tile rows [32v, 32v + 32)
constexpr int kBM = 128;       // tile rows (GEMM M)
constexpr int kBK = 64;        // K per LDS stage
constexpr int kLdk = kBK + 8;  // LDS row stride (bf16) of the operand tiles: 144 B, conflict-free 16-byte row reads

// Groups per tile: BN = TG*W columns of w (a multiple of 16 for any W <= 8).
constexpr int gen_tg(int W) { return W <= 4 ? 32 : 16; }

// Global -> register -> LDS staging of one operand tile of BR rows (rows of A
// or columns of B) by kBK k, stored K-contiguous in LDS ([BR][kLdk] bf16).
// KC: element (r, k) sits at p[r*ld + k] (k contiguous, K % 8 == 0); else at
// p[k*ld + r] (r contiguous, rows % 8 == 0): a thread then reads 8 rows at 4
// consecutive k and transposes them in registers.  Out-of-range elements are
// zero.
template <int BR, bool KC>
struct TileLoader {
    static constexpr int kUnits = KC ? BR * (kBK / 8) : (BR / 8) * (kBK / 4);
    static constexpr int kPer = (kUnits + kGBlock - 1) / kGBlock;
    static constexpr int kRegs = KC ? kPer : 4 * kPer;
    uint4 v[kRegs];

    __device__ __forceinline__ void load(const uint16_t *p, int64_t ld, int64_t rows, int64_t K, int64_t r0,
                                         int64_t k0, int tid) {
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int u = tid + i * kGBlock;
            if constexpr (KC) {
                const int64_t gr = r0 + (u >> 3), gk = k0 + (u & 7) * 8;
                v[i] = (u < kUnits && gr < rows && gk < K) ? *reinterpret_cast<const uint4 *>(p + gr * ld + gk)
                                                           : zero;
            } else {
                const int64_t gr = r0 + (u % (BR / 8)) * 8, gk = k0 + (u / (BR / 8)) * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[4 * i + j] = (u < kUnits && gr < rows && gk + j < K)
                                       ? *reinterpret_cast<const uint4 *>(p + (gk + j) * ld + gr)
                                       : zero;
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int u = tid + i * kGBlock;
            if (u >= kUnits) break;
            if constexpr (KC) {
                *reinterpret_cast<uint4 *>(lds + (u >> 3) * kLdk + (u & 7) * 8) = v[i];
            } else {
                const int rc = (u % (BR / 8)) * 8, kq = (u / (BR / 8)) * 4;
                const uint32_t w[4][4] = {{v[4 * i].x, v[4 * i].y, v[4 * i].z, v[4 * i].w},
                                          {v[4 * i + 1].x, v[4 * i + 1].y, v[4 * i + 1].z, v[4 * i + 1].w},
                                          {v[4 * i + 2].x, v[4 * i + 2].y, v[4 * i + 2].z, v[4 * i + 2].w},
                                          {v[4 * i + 3].x, v[4 * i + 3].y, v[4 * i + 3].z, v[4 * i + 3].w}};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // element e (row rc + e) of the four k rows
                    auto el = [&](int j) { return (w[j][e >> 1] >> (16 * (e & 1))) & 0xffffu; };
                    *reinterpret_cast<uint2 *>(lds + (rc + e) * kLdk + kq) =
                        make_uint2(el(0) | (el(1) << 16), el(2) | (el(3) << 16));
                }
            }
        }
    }
};

// C[kBM x BN] tile = A[m0 .., :] . B[n0 .., :]^T over the whole K, fp32 in
// registers: acc[mf][nf][j] is C[32v + 16mf + 4(lane>>4) + j][16nf + (lane&15)]
// for wave v.  `lds` holds two stages of both operand tiles.  Ends with a
// barrier, after which the LDS may be reused.
template <int BN, bool AKC, bool BKC>
__device__ __forceinline__ void gemm_tile(const uint16_t *A, int64_t lda, int64_t M, const uint16_t *B,
                                          int64_t ldb, int64_t Nc, int64_t K, int64_t m0, int64_t n0,
                                          uint16_t *lds, floatx4 (&acc)[2][BN / 16]) {
    constexpr int NF = BN / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint16_t *As[2] = {lds, lds + kBM * kLdk};
    uint16_t *Bs[2] = {lds + 2 * kBM * kLdk, lds + 2 * kBM * kLdk + BN * kLdk};
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = floatx4{0.f, 0.f, 0.f, 0.f};
    TileLoader<kBM, AKC> la;
    TileLoader<BN, BKC> lb;
    const int64_t nk = (K + kBK - 1) / kBK;
    la.load(A, lda, M, K, m0, 0, tid);
    lb.load(B, ldb, Nc, K, n0, 0, tid);
    la.store(As[0], tid);
    lb.store(Bs[0], tid);
    __syncthreads();
    const int arow = 32 * wave + (lane & 15), kofs = 8 * (lane >> 4);
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) {
            la.load(A, lda, M, K, m0, (kt + 1) * kBK, tid);
            lb.load(B, ldb, Nc, K, n0, (kt + 1) * kBK, tid);
        }
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8 a[2], b[NF];
#pragma unroll
            for (int mf = 0; mf < 2; ++mf)
                a[mf] = *reinterpret_cast<const bf16x8 *>(As[cur] + (arow + 16 * mf) * kLdk + kk + kofs);
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
                b[nf] = *reinterpret_cast<const bf16x8 *>(Bs[cur] + (16 * nf + (lane & 15)) * kLdk + kk + kofs);
#pragma unroll
            for (int mf = 0; mf < 2; ++mf)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf)
                    acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mf], b[nf], acc[mf][nf], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            la.store(As[cur ^ 1], tid);
            lb.store(Bs[cur ^ 1], tid);
        }
        __syncthreads();
    }
}

template <int BN>
constexpr int gemm_lds_bytes() {
    return 2 * (kBM + BN) * kLdk * 2;
}

// The accumulators into an fp32 LDS tile [kBM][BN + 4].
template <int BN>
__device__ __forceinline__ void park(const floatx4 (&acc)[2][BN / 16], float *Cs) {
    constexpr int ld = BN + 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int nf = 0; nf < BN / 16; ++nf)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Cs[(32 * wave + 16 * mf + 4 * (lane >> 4) + j) * ld + 16 * nf + (lane & 15)] = acc[mf][nf][j];
}

struct GenParams {
    const uint16_t *h, *V, *x, *dy;
    uint16_t *y, *dx, *dw;
    SeqMap seq;
    int64_t N, D, K, G;
    int32_t H;
    float rho;
    int64_t ntiles_n, ntiles_g;  // token tiles, group tiles
};

__device__ __forceinline__ void load8(const uint16_t *p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ void store8(uint16_t *p, const float (&v)[8]) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

__device__ __forceinline__ float ld_bf16(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }

// Forward: block = (token tile, group tile), walked so that the group tiles
// of one token tile (which share its rows of h) run on one XCD.
template <int W>
__global__ __launch_bounds__(kGBlock) void gen_fwd_kernel(GenParams p) {
    constexpr int TG = gen_tg(W), BN = TG * W, LDC = BN + 4;
    constexpr int kLds = gemm_lds_bytes<BN>() > kBM * LDC * 4 ? gemm_lds_bytes<BN>() : kBM * LDC * 4;
    __shared__ __align__(16) unsigned char lds[kLds];
    __shared__ int64_t seq_start[kBM];
    const int64_t lb = xcd_block_id(blockIdx.x, (int64_t)gridDim.x);
    const int64_t tn = lb / p.ntiles_g, tg = lb - tn * p.ntiles_g;
    const int64_t n0 = tn * kBM, g0 = tg * TG;
    const int tid = threadIdx.x;
    if (tid < kBM && n0 + tid < p.N) {
        int64_t s, e;
        p.seq.find(n0 + tid, s, e);
        seq_start[tid] = s;
    }
    floatx4 acc[2][BN / 16];
    gemm_tile<BN, true, true>(p.h, p.K, p.N, p.V, p.K, p.G * W, p.K, n0, g0 * W,
                              reinterpret_cast<uint16_t *>(lds), acc);
    float *Cs = reinterpret_cast<float *>(lds);
    park<BN>(acc, Cs);
    __syncthreads();

    // y of the tile's tokens over the channels of groups [g0, g0 + gcount):
    // one (token, 8-channel chunk) per item, consecutive threads along a row
    const int64_t gcount = min((int64_t)TG, p.G - g0);
    const int64_t c0 = g0 * p.H;
    const int nchunks = (int)(gcount * p.H / 8);
    const int64_t D = p.D;
    for (int it = tid; it < kBM * nchunks; it += kGBlock) {
        const int t = it / nchunks, q = it - t * nchunks;
        const int64_t n = n0 + t;
        if (n >= p.N) break;  // items are in token order
        const int64_t c = c0 + 8 * q;
        int col[8];  // the column of tap 0 of each channel's group in the tile
#pragma unroll
        for (int e = 0; e < 8; ++e) col[e] = (int)((c + e) / p.H - g0) * W;
        const float *wrow = Cs + t * LDC;
        float xv[8], out[8];
        load8(p.x + n * D + c, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(wrow[col[e]], xv[e], p.rho * xv[e]);
        const int64_t s = seq_start[t];
#pragma unroll
        for (int k = 1; k < W; ++k) {
            if (n - k < s) break;
            float xk[8];
            load8(p.x + (n - k) * D + c, xk);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(wrow[col[e] + k], xk[e], out[e]);
        }
        store8(p.y + n * D + c, out);
    }
}

// Backward, w recomputed: tile rows [n0, n0 + kBM) with n0 = tile * kStep;
// dx and dw of tokens [n0, n0 + kStep).  One (token, group) per item, so a
// group's filter gradient is summed in registers; VEC = 8 channels per load
// when H % 8 == 0, else one.
template <int W, int VEC>
__global__ __launch_bounds__(kGBlock) void gen_bwd_kernel(GenParams p) {
    constexpr int TG = gen_tg(W), BN = TG * W, LDC = BN + 4;
    constexpr int kStep = kBM - (W - 1);
    constexpr int kLds = gemm_lds_bytes<BN>() > kBM * LDC * 4 ? gemm_lds_bytes<BN>() : kBM * LDC * 4;
    __shared__ __align__(16) unsigned char lds[kLds];
    __shared__ int64_t seq_start[kBM], seq_end[kBM];
    const int64_t lb = xcd_block_id(blockIdx.x, (int64_t)gridDim.x);
    const int64_t tn = lb / p.ntiles_g, tg = lb - tn * p.ntiles_g;
    const int64_t n0 = tn * kStep, g0 = tg * TG;
    const int tid = threadIdx.x;
    if (tid < kStep && n0 + tid < p.N) {
        int64_t s, e;
        p.seq.find(n0 + tid, s, e);
        seq_start[tid] = s;
        seq_end[tid] = e;
    }
    floatx4 acc[2][BN / 16];
    gemm_tile<BN, true, true>(p.h, p.K, p.N, p.V, p.K, p.G * W, p.K, n0, g0 * W,
                              reinterpret_cast<uint16_t *>(lds), acc);
    float *Cs = reinterpret_cast<float *>(lds);
    park<BN>(acc, Cs);
    __syncthreads();

    const int gcount = (int)min((int64_t)TG, p.G - g0);
    const int64_t D = p.D, GW = p.G * W;
    const int H = p.H;
    for (int it = tid; it < kStep * gcount; it += kGBlock) {
        const int t = it / gcount, gl = it - t * gcount;
        const int64_t m = n0 + t;
        if (m >= p.N) break;
        const int64_t s = seq_start[t], e = seq_end[t];
        // taps whose token stays in m's sequence: dx reads m+k (k < ahead), dw reads m-k (k < back)
        const int ahead = (int)min((int64_t)W, e - m), back = (int)min((int64_t)W, m - s + 1);
        float wk[W];
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k] = k < ahead ? Cs[(t + k) * LDC + gl * W + k] : 0.f;
        float dws[W];
#pragma unroll
        for (int k = 0; k < W; ++k) dws[k] = 0.f;
        const int64_t cg = (g0 + gl) * H;
        for (int j = 0; j < H; j += VEC) {
            const int64_t c = cg + j;
            float gm[VEC], out[VEC];
            if constexpr (VEC == 8) load8(p.dy + m * D + c, gm);
            else gm[0] = ld_bf16(p.dy + m * D + c);
#pragma unroll
            for (int i = 0; i < VEC; ++i) out[i] = __builtin_fmaf(wk[0], gm[i], p.rho * gm[i]);
#pragma unroll
            for (int k = 1; k < W; ++k) {
                if (k >= ahead) break;
                float gk[VEC];
                if constexpr (VEC == 8) load8(p.dy + (m + k) * D + c, gk);
                else gk[0] = ld_bf16(p.dy + (m + k) * D + c);
#pragma unroll
                for (int i = 0; i < VEC; ++i) out[i] = __builtin_fmaf(wk[k], gk[i], out[i]);
            }
            if constexpr (VEC == 8) store8(p.dx + m * D + c, out);
            else p.dx[m * D + c] = to_bf16(out[0]);
#pragma unroll
            for (int k = 0; k < W; ++k) {
                if (k >= back) break;
                float xk[VEC];
                if constexpr (VEC == 8) load8(p.x + (m - k) * D + c, xk);
                else xk[0] = ld_bf16(p.x + (m - k) * D + c);
#pragma unroll
                for (int i = 0; i < VEC; ++i) dws[k] = __builtin_fmaf(gm[i], xk[i], dws[k]);
            }
        }
        uint16_t *dst = p.dw + m * GW + (g0 + gl) * W;
#pragma unroll
        for (int k = 0; k < W; ++k) dst[k] = to_bf16(dws[k]);
    }
}

// Plain product C (M x Nc) = A . B^T with an fp32 or bf16 store.
template <bool AKC, bool BKC, class OUT>
__global__ __launch_bounds__(kGBlock) void gemm_kernel(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                                                       int64_t M, int64_t Nc, int64_t K, OUT *C, int64_t ldc,
                                                       int64_t ntiles_n) {
    constexpr int BN = 128;
    __shared__ __align__(16) unsigned char lds[gemm_lds_bytes<BN>()];
    const int64_t lb = xcd_block_id(blockIdx.x, (int64_t)gridDim.x);
    const int64_t tm = lb / ntiles_n, tn = lb - tm * ntiles_n;
    const int64_t m0 = tm * kBM, n0 = tn * BN;
    floatx4 acc[2][BN / 16];
    gemm_tile<BN, AKC, BKC>(A, lda, M, B, ldb, Nc, K, m0, n0, reinterpret_cast<uint16_t *>(lds), acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int nf = 0; nf < BN / 16; ++nf) {
            const int64_t col = n0 + 16 * nf + (lane & 15);
            if (col >= Nc) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = m0 + 32 * wave + 16 * mf + 4 * (lane >> 4) + j;
                if (row >= M) continue;
                if constexpr (sizeof(OUT) == 4) C[row * ldc + col] = acc[mf][nf][j];
                else C[row * ldc + col] = to_bf16(acc[mf][nf][j]);
            }
        }
}

GenParams make_gen(const GenProblem &pr, int64_t tiles_n, int64_t tiles_g) {
    GenParams p;
    p.h = static_cast<const uint16_t *>(pr.h);
    p.V = static_cast<const uint16_t *>(pr.V);
    p.x = static_cast<const uint16_t *>(pr.x);
    p.dy = static_cast<const uint16_t *>(pr.dy);
    p.y = static_cast<uint16_t *>(pr.y);
    p.dx = static_cast<uint16_t *>(pr.dx);
    p.dw = static_cast<uint16_t *>(pr.dw);
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N;
    p.D = pr.D;
    p.K = pr.K;
    p.G = pr.D / pr.H;
    p.H = pr.H;
    p.rho = pr.residual ? 1.f : 0.f;
    p.ntiles_n = tiles_n;
    p.ntiles_g = tiles_g;
    return p;
}

template <int W>
hipError_t gen_fwd_w(const GenProblem &pr, hipStream_t st) {
    constexpr int TG = gen_tg(W);
    const int64_t G = pr.D / pr.H;
    const int64_t tn = (pr.N + kBM - 1) / kBM, tg = (G + TG - 1) / TG;
    const GenParams p = make_gen(pr, tn, tg);
    hipLaunchKernelGGL((gen_fwd_kernel<W>), dim3((unsigned)(tn * tg)), dim3(kGBlock), 0, st, p);
    return hipGetLastError();
}

template <int W>
hipError_t gen_bwd_w(const GenProblem &pr, hipStream_t st) {
    constexpr int TG = gen_tg(W);
    constexpr int kStep = kBM - (W - 1);
    const int64_t G = pr.D / pr.H, GW = G * W;
    const int64_t tn = (pr.N + kStep - 1) / kStep, tg = (G + TG - 1) / TG;
    const GenParams p = make_gen(pr, tn, tg);
    if (pr.H % 8 == 0)
        hipLaunchKernelGGL((gen_bwd_kernel<W, 8>), dim3((unsigned)(tn * tg)), dim3(kGBlock), 0, st, p);
    else
        hipLaunchKernelGGL((gen_bwd_kernel<W, 1>), dim3((unsigned)(tn * tg)), dim3(kGBlock), 0, st, p);
    // dh (N x K) = dw (N x GW, k contiguous) . V (GW x K, read as K-major columns)
    {
        const int64_t tm = (pr.N + kBM - 1) / kBM, tk = (pr.K + 127) / 128;
        hipLaunchKernelGGL((gemm_kernel<true, false, uint16_t>), dim3((unsigned)(tm * tk)), dim3(kGBlock), 0, st,
                           p.dw, GW, p.V, pr.K, pr.N, pr.K, GW, static_cast<uint16_t *>(pr.dh), pr.K, tk);
    }
    // dV (GW x K) = dw^T (rows contiguous along GW) . h (rows contiguous along K), summed over the N tokens
    {
        const int64_t tm = (GW + kBM - 1) / kBM, tk = (pr.K + 127) / 128;
        hipLaunchKernelGGL((gemm_kernel<false, false, float>), dim3((unsigned)(tm * tk)), dim3(kGBlock), 0, st,
                           p.dw, GW, p.h, pr.K, GW, pr.K, pr.N, pr.dV, pr.K, tk);
    }
    return hipGetLastError();
}

#define DSC_GEN_W_SWITCH(W_, CALL)                      \
    switch (W_) {                                       \
        case 1: { constexpr int Wc = 1; return CALL; }  \
        case 2: { constexpr int Wc = 2; return CALL; }  \
        case 3: { constexpr int Wc = 3; return CALL; }  \
        case 4: { constexpr int Wc = 4; return CALL; }  \
        case 5: { constexpr int Wc = 5; return CALL; }  \
        case 6: { constexpr int Wc = 6; return CALL; }  \
        case 7: { constexpr int Wc = 7; return CALL; }  \
        case 8: { constexpr int Wc = 8; return CALL; }  \
        default: return hipErrorInvalidValue;           \
    }

}  // namespace

hipError_t headwise_gen_fwd(const GenProblem &p, hipStream_t s) { DSC_GEN_W_SWITCH(p.W, gen_fwd_w<Wc>(p, s)); }

hipError_t headwise_gen_bwd(const GenProblem &p, hipStream_t s) { DSC_GEN_W_SWITCH(p.W, gen_bwd_w<Wc>(p, s)); }

}  // namespace dsc
