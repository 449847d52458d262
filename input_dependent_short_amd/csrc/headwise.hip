// headwise.hip -- head-wise tied dynamic short convolution, forward and
// backward, for gfx950.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: mechanism, parametrization (2) head-wise
// tying, placement with residual):
//   y[n,d] = rho*x[n,d] + sum_{k<W, n-k in seq(n)} w[n, d/H, k] * x[n-k, d]
// Backward for L = <dy, y>:
//   dx[m,d]   = rho*dy[m,d] + sum_{k<W, m+k in seq(m)} w[m+k, d/H, k] * dy[m+k, d]
//   dw[n,j,k] = [n-k in seq(n)] * sum_{d in group j} dy[n,d] * x[n-k, d]
//
// Design (HBM-bound streaming, about 2 FLOP per byte):
//   * one thread owns a 16-byte chunk of channels (8 bf16 / 4 fp32) and walks
//     a tile of TT consecutive tokens, so x, w and dy are each read once from
//     HBM and y, dx, dw written once; the W-1 token halo at each tile edge is
//     re-read and mostly hits L2 (neighbouring tiles run on the same XCD);
//   * the causal window is a register ring of the last W-1 inputs (forward)
//     plus a W-1 token look-ahead of (dy, w) in the backward;
//   * consecutive lanes own consecutive chunks of one token row, so every
//     wave access is a contiguous run of 16-byte vectors;
//   * taps outside the token's sequence are masked per token, so packed
//     sequences cost nothing when no boundary falls inside a tile;
//   * the dw group sum over H channels is a per-thread sum over the chunk
//     followed by a butterfly over the H/VEC lanes of the group;
//   * fp32 accumulation, one round-to-nearest-even store per output.
#include "dsc_kernels.h"

namespace dsc {
namespace {

struct HwParams {
    const void *x, *w, *dy;
    void *y, *dx, *dw;
    SeqMap seq;
    int64_t N, D, G;
    int32_t H;
    int32_t lanes;  // lanes sharing one filter group (H / VEC when H >= VEC)
    float rho;
    int64_t nchunks, items;
};

constexpr int kBlock = 256;

// Group-local index of channel c of a chunk in the thread's filter span.
template <int VEC, int GPT>
__device__ __forceinline__ constexpr int grp(int c) {
    return GPT > 1 ? c / (VEC / GPT) : 0;
}

template <class E, int W, int GPT, int TT, int U>
__global__ __launch_bounds__(kBlock) void hw_fwd_kernel(HwParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int NW = GPT * W;
    constexpr int WALIGN = pow2_align(NW * (int)sizeof(S));

    const int64_t item = xcd_block_id(blockIdx.x, gridDim.x) * kBlock + threadIdx.x;
    if (item >= p.items) return;
    const int64_t tile = item / p.nchunks;
    const int64_t chunk = item - tile * p.nchunks;
    const int64_t n0 = tile * TT;
    const int64_t n1 = min(n0 + (int64_t)TT, p.N);
    const int64_t d0 = chunk * VEC;
    const int64_t jfirst = GPT > 1 ? chunk * GPT : d0 / p.H;

    const S *x = static_cast<const S *>(p.x) + d0;
    const S *w = static_cast<const S *>(p.w) + jfirst * W;
    S *y = static_cast<S *>(p.y) + d0;

    int64_t s, e;
    p.seq.find(n0, s, e);

    // ring[i] holds x[n-1-i]
    float ring[W > 1 ? W - 1 : 1][VEC];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int64_t t = n0 - 1 - i;
        if (t >= s) {
            Vec16<E>::load(x + t * p.D, ring[i]);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) ring[i][c] = 0.f;
        }
    }

    for (int64_t nb = n0; nb < n1; nb += U) {
        float xv[U][VEC];
        float wv[U][NW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = nb + u;
            if (n < n1) {
                Vec16<E>::load(x + n * p.D, xv[u]);
                Span<E, NW>::template load<WALIGN>(w + n * p.G * W, wv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = nb + u;
            if (n < n1) {
                if (n >= e) p.seq.find(n, s, e);
                const int64_t nv = n - s;  // taps k <= nv lie inside the sequence
                float acc[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = p.rho * xv[u][c];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const bool ok = k <= nv;
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        const float wk = ok ? wv[u][grp<VEC, GPT>(c) * W + k] : 0.f;
                        const float xk = k == 0 ? xv[u][c] : ring[k - 1][c];
                        acc[c] = __builtin_fmaf(wk, xk, acc[c]);
                    }
                }
                Vec16<E>::store(y + n * p.D, acc);
#pragma unroll
                for (int i = W - 2; i > 0; --i)
#pragma unroll
                    for (int c = 0; c < VEC; ++c) ring[i][c] = ring[i - 1][c];
                if constexpr (W > 1) {
#pragma unroll
                    for (int c = 0; c < VEC; ++c) ring[0][c] = xv[u][c];
                }
            }
        }
    }
}

template <class E, int W, int GPT, int TT, int U>
__global__ __launch_bounds__(kBlock) void hw_bwd_kernel(HwParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int NW = GPT * W;
    constexpr int WALIGN = pow2_align(NW * (int)sizeof(S));
    constexpr int WIN = U + W - 1;  // look-ahead window of (dy, w)

    const int64_t item = xcd_block_id(blockIdx.x, gridDim.x) * kBlock + threadIdx.x;
    // Whole filter groups are active or inactive together (items is a
    // multiple of nchunks, which is a multiple of lanes), so exiting here never
    // strands a lane that a group butterfly reads.
    if (item >= p.items) return;
    const int64_t tile = item / p.nchunks;
    const int64_t chunk = item - tile * p.nchunks;
    const int64_t n0 = tile * TT;
    const int64_t n1 = min(n0 + (int64_t)TT, p.N);
    const int64_t d0 = chunk * VEC;
    const int64_t jfirst = GPT > 1 ? chunk * GPT : d0 / p.H;
    const bool leader = (chunk & (p.lanes - 1)) == 0;

    const S *x = static_cast<const S *>(p.x) + d0;
    const S *g = static_cast<const S *>(p.dy) + d0;
    const S *w = static_cast<const S *>(p.w) + jfirst * W;
    S *dx = static_cast<S *>(p.dx) + d0;
    S *dw = static_cast<S *>(p.dw) + jfirst * W;

    int64_t s, e;
    p.seq.find(n0, s, e);

    float ring[W > 1 ? W - 1 : 1][VEC];  // ring[i] = x[m-1-i]
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int64_t t = n0 - 1 - i;
        if (t >= s) {
            Vec16<E>::load(x + t * p.D, ring[i]);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) ring[i][c] = 0.f;
        }
    }
    // window slot i holds token mb + i
    float gw[WIN][VEC];
    float ww[WIN][NW];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int64_t t = n0 + i;
        if (t < p.N) {
            Vec16<E>::load(g + t * p.D, gw[i]);
            Span<E, NW>::template load<WALIGN>(w + t * p.G * W, ww[i]);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) gw[i][c] = 0.f;
#pragma unroll
            for (int c = 0; c < NW; ++c) ww[i][c] = 0.f;
        }
    }

    for (int64_t mb = n0; mb < n1; mb += U) {
        float xv[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t m = mb + u;
            if (m < n1) Vec16<E>::load(x + m * p.D, xv[u]);
            const int64_t t = mb + W - 1 + u;
            if (t < p.N) {
                Vec16<E>::load(g + t * p.D, gw[W - 1 + u]);
                Span<E, NW>::template load<WALIGN>(w + t * p.G * W, ww[W - 1 + u]);
            } else {
#pragma unroll
                for (int c = 0; c < VEC; ++c) gw[W - 1 + u][c] = 0.f;
#pragma unroll
                for (int c = 0; c < NW; ++c) ww[W - 1 + u][c] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t m = mb + u;
            if (m < n1) {
                if (m >= e) p.seq.find(m, s, e);
                const int64_t ahead = e - m;  // dx terms k < ahead stay in the sequence
                const int64_t back = m - s;   // dw taps k <= back stay in the sequence
                float acc[VEC];
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = p.rho * gw[u][c];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const bool ok = k < ahead;
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        const float wk = ok ? ww[u + k][grp<VEC, GPT>(c) * W + k] : 0.f;
                        acc[c] = __builtin_fmaf(wk, gw[u + k][c], acc[c]);
                    }
                }
                Vec16<E>::store(dx + m * p.D, acc);

                float part[NW];
#pragma unroll
                for (int i = 0; i < NW; ++i) part[i] = 0.f;
#pragma unroll
                for (int k = 0; k < W; ++k) {
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        const float xk = k == 0 ? xv[u][c] : ring[k - 1][c];
                        part[grp<VEC, GPT>(c) * W + k] =
                            __builtin_fmaf(gw[u][c], xk, part[grp<VEC, GPT>(c) * W + k]);
                    }
                }
                for (int off = 1; off < p.lanes; off <<= 1) {
#pragma unroll
                    for (int i = 0; i < NW; ++i) part[i] += __shfl_xor(part[i], off, kWave);
                }
#pragma unroll
                for (int q = 0; q < GPT; ++q)
#pragma unroll
                    for (int k = 0; k < W; ++k)
                        if (k > back) part[q * W + k] = 0.f;
                if (leader) Span<E, NW>::template store<WALIGN>(dw + m * p.G * W, part);

#pragma unroll
                for (int i = W - 2; i > 0; --i)
#pragma unroll
                    for (int c = 0; c < VEC; ++c) ring[i][c] = ring[i - 1][c];
                if constexpr (W > 1) {
#pragma unroll
                    for (int c = 0; c < VEC; ++c) ring[0][c] = xv[u][c];
                }
            }
        }
        // slide the look-ahead window by U tokens
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) gw[i][c] = gw[U + i][c];
#pragma unroll
            for (int c = 0; c < NW; ++c) ww[i][c] = ww[U + i][c];
        }
    }
}

constexpr int kTT = 32;  // tokens per thread tile
constexpr int kU = 4;    // tokens per load batch

template <class E>
HwParams make_params(const HwProblem &pr, int64_t &blocks) {
    HwParams p;
    p.x = pr.x; p.w = pr.w; p.dy = pr.dy;
    p.y = pr.y; p.dx = pr.dx; p.dw = pr.dw;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N; p.D = pr.D; p.G = pr.D / pr.H;
    p.H = pr.H;
    p.lanes = pr.H >= E::kVec ? pr.H / E::kVec : 1;
    p.rho = pr.residual ? 1.f : 0.f;
    p.nchunks = pr.D / E::kVec;
    const int64_t ntiles = (pr.N + kTT - 1) / kTT;
    p.items = ntiles * p.nchunks;
    blocks = (p.items + kBlock - 1) / kBlock;
    return p;
}

template <class E, int W, int GPT>
hipError_t launch_w(const HwProblem &pr, hipStream_t st, bool bwd) {
    int64_t blocks;
    HwParams p = make_params<E>(pr, blocks);
    if (blocks == 0) return hipSuccess;
    if (bwd)
        hipLaunchKernelGGL((hw_bwd_kernel<E, W, GPT, kTT, kU>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
    else
        hipLaunchKernelGGL((hw_fwd_kernel<E, W, GPT, kTT, kU>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
    return hipGetLastError();
}

template <class E, int GPT>
hipError_t dispatch_w(const HwProblem &pr, hipStream_t st, bool bwd) {
    switch (pr.W) {
        case 1: return launch_w<E, 1, GPT>(pr, st, bwd);
        case 2: return launch_w<E, 2, GPT>(pr, st, bwd);
        case 3: return launch_w<E, 3, GPT>(pr, st, bwd);
        case 4: return launch_w<E, 4, GPT>(pr, st, bwd);
        case 5: return launch_w<E, 5, GPT>(pr, st, bwd);
        case 6: return launch_w<E, 6, GPT>(pr, st, bwd);
        case 7: return launch_w<E, 7, GPT>(pr, st, bwd);
        case 8: return launch_w<E, 8, GPT>(pr, st, bwd);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
hipError_t dispatch(const HwProblem &pr, hipStream_t st, bool bwd) {
    constexpr int VEC = E::kVec;
    if (pr.H >= VEC) return dispatch_w<E, 1>(pr, st, bwd);
    switch (VEC / pr.H) {
        case 2: return dispatch_w<E, 2>(pr, st, bwd);
        case 4: return dispatch_w<E, 4>(pr, st, bwd);
        case 8:
            if constexpr (VEC >= 8) return dispatch_w<E, 8>(pr, st, bwd);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool headwise_supported(Dtype dt, int64_t D, int32_t H) {
    const int VEC = dt == Dtype::BF16 ? BF16::kVec : F32::kVec;
    if (H < 1 || D % H) return false;
    if (H < VEC) return VEC % H == 0;
    const int lanes = H / VEC;
    return H % VEC == 0 && (lanes & (lanes - 1)) == 0 && lanes <= kWave;
}

hipError_t headwise_fwd(const HwProblem &p, hipStream_t s) {
    return p.dtype == Dtype::BF16 ? dispatch<BF16>(p, s, false) : dispatch<F32>(p, s, false);
}

hipError_t headwise_bwd(const HwProblem &p, hipStream_t s) {
    return p.dtype == Dtype::BF16 ? dispatch<BF16>(p, s, true) : dispatch<F32>(p, s, true);
}

}  // namespace dsc
