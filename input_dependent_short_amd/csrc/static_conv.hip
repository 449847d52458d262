// static_conv.hip -- the static short convolution for gfx950: one filter per
// channel, the same at every position.  It is the layer that the dynamic
// convolution generalises, and its optimised kernels are what the pages set
// the dynamic kernels' latency against (gist.science technical summary,
// Performance; the authors' thread on digg.com describes it as a depthwise
// causal convolution of small width):
//   y[n,d]  = rho*x[n,d] + sum_{k<W, n-k in seq(n)} c[d,k] * x[n-k,d]
// Backward for L = <dy, y>:
//   dx[m,d] = rho*dy[m,d] + sum_{k<W, m+k in seq(m)} c[d,k] * dy[m+k,d]
//   dc[d,k] = sum_n [n-k in seq(n)] dy[n,d] * x[n-k,d]
//
// Design (HBM-bound streaming, the head-wise layout with the filter read once):
//   * one thread owns a 16-byte channel chunk (8 bf16 / 4 fp32) and walks a
//     tile of consecutive tokens; consecutive lanes take consecutive chunks of
//     one token row, so every wave access is a contiguous run of 16-byte
//     vectors;
//   * the chunk's W filter taps are loaded once into registers, with rho
//     folded into tap 0;
//   * the causal window is a register ring of the last W-1 inputs that is
//     cleared when the walk enters a new sequence, so taps reaching before a
//     sequence start read zeros and need no per-tap masks; only the
//     backward's look-ahead near a sequence end masks taps (a uniform branch);
//   * dc is a sum over every token: each thread sums its tile, a block (up to
//     64 chunks x the consecutive tiles its 256 threads cover) adds the
//     partials in LDS and issues one fp32 atomic per (channel, tap), after a
//     zero-fill launch (the only launch of an empty batch).
#include "dsc_kernels.h"

namespace dsc {
namespace {

struct StParams {
    const void *x, *c, *dy;
    void *y, *dx;
    float *dc;
    SeqMap seq;
    int64_t N, D;
    float rho;
    int64_t nchunks;  // 16-byte channel chunks per token row
    int64_t items;    // forward: threads with work (tiles x chunks)
    int64_t ntiles;   // token tiles
    int64_t ncg;      // backward: groups of cb chunks
    int32_t cb;       // backward: chunks per block (power of two, 8..64)
    int64_t dc_stride;  // backward: dc of token-tile group q goes to dc + q*dc_stride (0: one sum)
};

constexpr int kBlock = 256;

template <class E>
__device__ __forceinline__ void load_vec(const typename E::store_t *p, float (&v)[E::kVec]) {
    Vec16<E>::load(p, v);
}

// The W taps of VEC consecutive channels (VEC*W contiguous elements of the
// (D, W) filter, 16-byte aligned), with rho added to tap 0.
template <class E, int W>
__device__ __forceinline__ void load_taps(const typename E::store_t *c, float rho, float (&cf)[E::kVec][W]) {
    constexpr int VEC = E::kVec;
    float v[VEC];
#pragma unroll
    for (int q = 0; q < W; ++q) {  // W 16-byte vectors hold the VEC*W taps
        load_vec<E>(c + q * VEC, v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const int e = q * VEC + i;
            cf[e / W][e % W] = v[i];
        }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) cf[i][0] += rho;
}

// Element c of a raw 16-byte vector, widened to fp32.
template <class E>
__device__ __forceinline__ float elem(const uint4 &v, int c) {
    constexpr int PW = E::kVec / 4;  // elements per 32-bit word
    const uint32_t w = c < PW ? v.x : c < 2 * PW ? v.y : c < 3 * PW ? v.z : v.w;
    if constexpr (PW == 1) {
        return __uint_as_float(w);
    } else {
        return (c & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

// Forward: thread = (tile of TT tokens, chunk); batches of U tokens are
// loaded one batch ahead of the arithmetic.
template <class E, int W, int TT, int U>
__global__ __launch_bounds__(kBlock) void st_fwd_kernel(StParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int RW = W > 1 ? W - 1 : 1;

    const int64_t item = xcd_block_id(blockIdx.x, gridDim.x) * kBlock + threadIdx.x;
    if (item >= p.items) return;
    const int64_t tile = item / p.nchunks;
    const int64_t chunk = item - tile * p.nchunks;
    const int64_t n0 = tile * TT;
    const int64_t n1 = min(n0 + (int64_t)TT, p.N);
    const int64_t d0 = chunk * VEC;
    const S *x = static_cast<const S *>(p.x) + d0;
    S *y = static_cast<S *>(p.y) + d0;

    float cf[VEC][W];
    load_taps<E, W>(static_cast<const S *>(p.c) + d0 * W, p.rho, cf);

    int64_t s, e;
    p.seq.find(n0, s, e);
    // inputs stay raw 16-byte rows until used (widened per use)
    uint4 ring[RW];  // ring[i] = x[n-1-i], zero before n's sequence
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int64_t t = n0 - 1 - i;
        ring[i] = make_uint4(0u, 0u, 0u, 0u);
        if (t >= s) ring[i] = *reinterpret_cast<const uint4 *>(x + t * p.D);
    }

    uint4 xa[U], xb[U];
    auto load_batch = [&](int64_t nb, uint4 (&xr)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (nb + u < n1) xr[u] = *reinterpret_cast<const uint4 *>(x + (nb + u) * p.D);
    };
    auto compute_batch = [&](int64_t nb, const uint4 (&xr)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = nb + u;
            if (n < n1) {
                if (n >= e) {  // n starts the next sequence: earlier inputs do not reach it
                    p.seq.find(n, s, e);
#pragma unroll
                    for (int i = 0; i < RW; ++i) ring[i] = make_uint4(0u, 0u, 0u, 0u);
                }
                float acc[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    float a = cf[c][0] * elem<E>(xr[u], c);
#pragma unroll
                    for (int k = 1; k < W; ++k) a = __builtin_fmaf(cf[c][k], elem<E>(ring[k - 1], c), a);
                    acc[c] = a;
                }
                Vec16<E>::store(y + n * p.D, acc);
#pragma unroll
                for (int i = W - 2; i > 0; --i) ring[i] = ring[i - 1];
                if constexpr (W > 1) ring[0] = xr[u];
            }
        }
    };

    load_batch(n0, xa);
    for (int64_t nb = n0; nb < n1; nb += 2 * U) {
        if (nb + U < n1) load_batch(nb + U, xb);
        compute_batch(nb, xa);
        if (nb + U >= n1) break;
        if (nb + 2 * U < n1) load_batch(nb + 2 * U, xa);
        compute_batch(nb + U, xb);
    }
}


constexpr int kRedFloats = 32 * (kBlock + kBlock / 8);  // LDS of the dc reduction, any chunks-per-block

// Backward: block = cb chunks (a power of two, 8..64, chosen so the row
// divides evenly when it can) x kBlock/cb consecutive tiles of TT tokens;
// thread (tile, chunk) walks the tile.  The dy look-ahead window and the x
// batch stay packed in registers and are widened where used, which keeps
// the kernel at 3 waves per SIMD.  Every thread reaches the block reduction
// of dc, with zero partials when it has no work.
template <class E, int W, int TT, int U>
__global__ __launch_bounds__(kBlock) void st_bwd_kernel(StParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int RW = W > 1 ? W - 1 : 1;
    constexpr int WIN = U + W - 1;                 // look-ahead window of dy
    constexpr int NE = VEC * W;                    // dc partials per thread
    constexpr int EC = NE <= 32 ? NE : NE / 2;     // partials per reduction round (NE is even)
    static_assert(NE % EC == 0 && EC <= 32, "whole reduction rounds that fit the LDS");
    __shared__ float red[kRedFloats];              // [tile][partial][chunk], odd chunk pitch

    const int cb = p.cb;
    const int tpb = kBlock / cb;
    const int cin = threadIdx.x & (cb - 1);
    const int tin = threadIdx.x / cb;
    const int64_t b = xcd_block_id(blockIdx.x, gridDim.x);
    const int64_t tq = b / p.ncg;
    const int64_t cg = b - tq * p.ncg;
    const int64_t chunk = cg * cb + cin;
    const int64_t tile = tq * tpb + tin;
    const bool active = chunk < p.nchunks && tile < p.ntiles;

    float part[VEC][W];
#pragma unroll
    for (int c = 0; c < VEC; ++c)
#pragma unroll
        for (int k = 0; k < W; ++k) part[c][k] = 0.f;

    if (active) {
        const int64_t n0 = tile * TT;
        const int64_t n1 = min(n0 + (int64_t)TT, p.N);
        const int64_t d0 = chunk * VEC;
        const S *x = static_cast<const S *>(p.x) + d0;
        const S *g = static_cast<const S *>(p.dy) + d0;
        S *dx = static_cast<S *>(p.dx) + d0;

        float cf[VEC][W];
        load_taps<E, W>(static_cast<const S *>(p.c) + d0 * W, p.rho, cf);

        int64_t s, e;
        p.seq.find(n0, s, e);
        // raw rows, widened where they are used: ring[i] = x[m-1-i], zero
        // before m's sequence
        uint4 ring[RW];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            const int64_t t = n0 - 1 - i;
            ring[i] = make_uint4(0u, 0u, 0u, 0u);
            if (t >= s) ring[i] = *reinterpret_cast<const uint4 *>(x + t * p.D);
        }
        // raw 16-byte rows, zero past the end (a branch, not a select between
        // addresses, so the load stays a global load)
        auto load_row = [&](const S *base, int64_t t, int64_t end) {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (t < end) v = *reinterpret_cast<const uint4 *>(base + t * p.D);
            return v;
        };
        uint4 gw[WIN];  // gw[i] = dy[mb + i] (zero past N)
        auto load_g = [&](int64_t t) { return load_row(g, t, p.N); };
#pragma unroll
        for (int i = 0; i < W - 1; ++i) gw[i] = load_g(n0 + i);

        for (int64_t mb = n0; mb < n1; mb += U) {
            uint4 xv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u] = load_row(x, mb + u, n1);
                gw[W - 1 + u] = load_g(mb + W - 1 + u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t m = mb + u;
                if (m < n1) {
                    if (m >= e) {  // m starts the next sequence
                        p.seq.find(m, s, e);
#pragma unroll
                        for (int i = 0; i < RW; ++i) ring[i] = make_uint4(0u, 0u, 0u, 0u);
                    }
                    // dx: taps k with m+k in m's sequence (all of them unless m is
                    // among its sequence's last W-1 tokens)
                    float acc[VEC];
                    if (e - m >= W) {
#pragma unroll
                        for (int c = 0; c < VEC; ++c) {
                            float a = cf[c][0] * elem<E>(gw[u], c);
#pragma unroll
                            for (int k = 1; k < W; ++k) a = __builtin_fmaf(cf[c][k], elem<E>(gw[u + k], c), a);
                            acc[c] = a;
                        }
                    } else {
                        const int64_t ahead = e - m;
#pragma unroll
                        for (int c = 0; c < VEC; ++c) {
                            float a = cf[c][0] * elem<E>(gw[u], c);
#pragma unroll
                            for (int k = 1; k < W; ++k)
                                a = __builtin_fmaf(k < ahead ? cf[c][k] : 0.f, elem<E>(gw[u + k], c), a);
                            acc[c] = a;
                        }
                    }
                    Vec16<E>::store(dx + m * p.D, acc);
                    // dc partials: dy[m] * x[m-k] (the ring reads zero before the sequence)
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        const float gv = elem<E>(gw[u], c), xc = elem<E>(xv[u], c);
                        part[c][0] = __builtin_fmaf(gv, xc, part[c][0]);
#pragma unroll
                        for (int k = 1; k < W; ++k) part[c][k] = __builtin_fmaf(gv, elem<E>(ring[k - 1], c), part[c][k]);
                    }
#pragma unroll
                    for (int i = W - 2; i > 0; --i) ring[i] = ring[i - 1];
                    if constexpr (W > 1) ring[0] = xv[u];
                }
            }
#pragma unroll
            for (int i = 0; i < W - 1; ++i) gw[i] = gw[U + i];
        }
    }

    // dc: the partials of each (chunk, tap) over the block's tiles summed in
    // LDS, one atomic per (channel, tap).  Partial e of a thread is dc element
    // chunk*NE + e (taps innermost), so a round's atomics run over contiguous
    // addresses.
    const int pitch = cb + 1;
#pragma unroll
    for (int r0 = 0; r0 < NE; r0 += EC) {
        if (r0) __syncthreads();  // the previous round's reads are done
#pragma unroll
        for (int i = 0; i < EC; ++i) red[(tin * EC + i) * pitch + cin] = part[(r0 + i) / W][(r0 + i) % W];
        __syncthreads();
        for (int j = threadIdx.x; j < cb * EC; j += kBlock) {
            const int cl = j / EC, i = j - cl * EC;
            float v = 0.f;
            for (int t = 0; t < tpb; ++t) v += red[(t * EC + i) * pitch + cl];
            const int64_t ch = cg * cb + cl;
            if (ch < p.nchunks) atomicAdd(p.dc + tq * p.dc_stride + ch * NE + r0 + i, v);
        }
    }
}

// dst[i] = src[i] + src[stride + i] + ... + src[(nparts-1)*stride + i], in that
// order: the fixed-order sum of the token-tile groups' dc regions.
__global__ __launch_bounds__(kBlock) void st_sum_parts(const float *src, int64_t nparts, int64_t stride, float *dst,
                                                       int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    float a = 0.f;
    // unrolled so that the loads of several regions are in flight together; the
    // additions keep the ascending order
#pragma unroll 16
    for (int64_t j = 0; j < nparts; ++j) a += src[j * stride + i];
    dst[i] = a;
}

// Zero-fills dc (n floats, 16-byte aligned) before the backward's atomics.
__global__ __launch_bounds__(kBlock) void st_zero(float *p, int64_t n) {
    const int64_t i = 4 * ((int64_t)blockIdx.x * kBlock + threadIdx.x);
    if (i + 3 < n) {
        *reinterpret_cast<float4 *>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        for (int64_t j = i; j < n; ++j) p[j] = 0.f;
    }
}

#ifndef DSC_ST_TT
#define DSC_ST_TT 32
#endif
constexpr int kStTT = DSC_ST_TT;  // tokens per thread tile
constexpr int kStU = 4;           // tokens per load batch (forward)
// tokens per load batch (backward): 4, or 2 where the W*VEC dc partials of a
// wider filter leave no room for the deeper batch
constexpr int st_bwd_batch(int W) { return W <= 4 ? 4 : 2; }

// Chunks per backward block: 64, or the largest of 32, 16, 8 that divides the
// row when 64 does not (no idle lanes), else 64 with a ragged last group.
int chunks_per_block(int64_t nchunks) {
    if (nchunks % kWave == 0) return kWave;
    for (int cb : {32, 16, 8})
        if (nchunks % cb == 0) return cb;
    return kWave;
}

template <class E>
StParams make_params(const StProblem &pr) {
    StParams p;
    p.x = pr.x; p.c = pr.c; p.dy = pr.dy;
    p.y = pr.y; p.dx = pr.dx; p.dc = pr.dc;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N; p.D = pr.D;
    p.rho = pr.residual ? 1.f : 0.f;
    p.nchunks = pr.D / E::kVec;
    p.ntiles = (pr.N + kStTT - 1) / kStTT;
    p.items = p.ntiles * p.nchunks;
    p.cb = chunks_per_block(p.nchunks);
    p.ncg = (p.nchunks + p.cb - 1) / p.cb;
    p.dc_stride = 0;
    return p;
}

// Token-tile groups of the backward (blocks along the token axis): the
// number of dc regions of the fixed-order backward.
int64_t tile_groups(int64_t N, int64_t nchunks) {
    const int64_t ntiles = (N + kStTT - 1) / kStTT;
    const int64_t tpb = kBlock / chunks_per_block(nchunks);
    return (ntiles + tpb - 1) / tpb;
}

// det_ws: the fixed-order backward's workspace (one dc region per token-tile
// group, summed in order after the kernel), or null for the atomics into dc.
template <class E, int W>
hipError_t launch(const StProblem &pr, hipStream_t st, bool bwd, float *det_ws = nullptr) {
    StParams p = make_params<E>(pr);
    if (!bwd) {
        const int64_t blocks = (p.items + kBlock - 1) / kBlock;
        if (blocks) hipLaunchKernelGGL((st_fwd_kernel<E, W, kStTT, kStU>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
        return hipGetLastError();
    }
    const int64_t nz = pr.D * pr.W;
    const int64_t nq = tile_groups(pr.N, p.nchunks);
    if (det_ws && nq > 0) {  // regions of their own, one per token-tile group
        p.dc = det_ws;
        p.dc_stride = nz;
    }
    const int64_t nclear = p.dc_stride ? nq * nz : nz;
    hipLaunchKernelGGL(st_zero, dim3((unsigned)((nclear + 4 * kBlock - 1) / (4 * kBlock))), dim3(kBlock), 0, st, p.dc,
                       nclear);
    const int64_t tpb = kBlock / p.cb;
    const int64_t blocks = (p.ntiles + tpb - 1) / tpb * p.ncg;  // none for an empty batch
    if (blocks)
        hipLaunchKernelGGL((st_bwd_kernel<E, W, kStTT, st_bwd_batch(W)>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
    if (p.dc_stride)
        hipLaunchKernelGGL(st_sum_parts, dim3((unsigned)((nz + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, p.dc, nq,
                           nz, pr.dc, nz);
    return hipGetLastError();
}

template <class E>
hipError_t dispatch(const StProblem &pr, hipStream_t st, bool bwd, float *det_ws = nullptr) {
    switch (pr.W) {
        case 1: return launch<E, 1>(pr, st, bwd, det_ws);
        case 2: return launch<E, 2>(pr, st, bwd, det_ws);
        case 3: return launch<E, 3>(pr, st, bwd, det_ws);
        case 4: return launch<E, 4>(pr, st, bwd, det_ws);
        case 5: return launch<E, 5>(pr, st, bwd, det_ws);
        case 6: return launch<E, 6>(pr, st, bwd, det_ws);
        case 7: return launch<E, 7>(pr, st, bwd, det_ws);
        case 8: return launch<E, 8>(pr, st, bwd, det_ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t static_fwd(const StProblem &p, hipStream_t s) {
    return p.dtype == Dtype::BF16 ? dispatch<BF16>(p, s, false) : dispatch<F32>(p, s, false);
}

hipError_t static_bwd(const StProblem &p, hipStream_t s) {
    return p.dtype == Dtype::BF16 ? dispatch<BF16>(p, s, true) : dispatch<F32>(p, s, true);
}

size_t static_bwd_det_workspace(Dtype dt, int64_t N, int64_t D, int32_t W) {
    const int64_t nchunks = D / (dt == Dtype::BF16 ? BF16::kVec : F32::kVec);
    if (N <= 0 || nchunks <= 0) return 0;
    const size_t bytes = (size_t)tile_groups(N, nchunks) * (size_t)D * W * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t static_bwd_det(const StProblem &p, float *ws, hipStream_t s) {
    return p.dtype == Dtype::BF16 ? dispatch<BF16>(p, s, true, ws) : dispatch<F32>(p, s, true, ws);
}

}  // namespace dsc
