// headwise_any.hip -- head-wise tied dynamic short convolution for any
// group size H (D % H == 0), for gfx950.  The kernels of headwise_impl.h
// assume that a 16-byte channel chunk holds whole filter groups or that a
// group covers a whole number of chunks on at most 64 lanes; these cover the
// rest (H = 3, 5, 6, 12, 20, ..., and groups wider than 64 chunks).
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: mechanism, parametrization (2) head-wise
// tying -- one filter shared by H consecutive channels, placement with
// residual), as in headwise_impl.h:
//   y[n,d]    = rho*x[n,d] + sum_{k<W, n-k in seq(n)} w[n, d/H, k] * x[n-k, d]
//   dx[m,d]   = rho*dy[m,d] + sum_{k<W, m+k in seq(m)} w[m+k, d/H, k] * dy[m+k, d]
//   dw[n,j,k] = [n-k in seq(n)] * sum_{d in group j} dy[n,d] * x[n-k, d]
// and with ROPE the rotary embedding of channels d < rot after the layer
// ("RoFormer: Enhanced Transformer with Rotary Position Embedding", Su et
// al., Section 3.4.2): the forward turns the output, the backward turns dy
// back first (ds = R^T dy) and runs the layer's backward on ds.
//
// Design (correct for every H, not tuned):
//   * forward and dx: one thread per (32-token tile, 16-byte channel chunk),
//     a register ring of the last W-1 inputs (forward); each channel of the
//     chunk reads the filter of its own group d/H;
//   * dw: the backward's dx and dw run as two launches; dw takes one segment
//     of P lanes (H rounded up to a power of two, at most 64) per (token,
//     filter group), each lane summing every P-th channel of the group, then a
//     butterfly over the segment's lanes.  dy and x are read once more than in
//     the fused kernels;
//   * cos / sin come from the table row of the token's position in its
//     sequence.
#include "dsc_kernels.h"

namespace dsc {
namespace {

constexpr int kAnyBlock = 256;
constexpr int kAnyTT = 32;  // tokens per thread tile (forward, dx)

struct AnyParams {
    const void *x, *w, *dy;
    void *y, *dx, *dw;
    SeqMap seq;
    int64_t N, D, G;
    int32_t H;
    float rho;
    int64_t nchunks, items;
    const float *rope;  // (npos, hd/2, 2) cos, sin; read only with ROPE
    int32_t rot, hd, npos;
    int32_t P;  // dw: lanes per (token, group) segment
};

template <class E>
__device__ __forceinline__ float elem(const typename E::store_t *p, int64_t i) {
    return load_elem<E>(p + i);
}

template <class E, int W, bool ROPE>
__global__ __launch_bounds__(kAnyBlock) void hw_any_fwd(AnyParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int WA = pow2_align(W * (int)sizeof(S));
    using WS = RawSpan<E, W>;
    const int64_t item = (int64_t)blockIdx.x * kAnyBlock + threadIdx.x;
    if (item >= p.items) return;
    const int64_t tile = item / p.nchunks;
    const int64_t chunk = item - tile * p.nchunks;
    const int64_t n0 = tile * kAnyTT;
    const int64_t n1 = min(n0 + (int64_t)kAnyTT, p.N);
    const int64_t d0 = chunk * VEC;
    const S *x = static_cast<const S *>(p.x) + d0;
    const S *w = static_cast<const S *>(p.w);
    S *y = static_cast<S *>(p.y) + d0;
    int64_t j[VEC];  // filter group of each channel of the chunk
#pragma unroll
    for (int c = 0; c < VEC; ++c) j[c] = (d0 + c) / p.H;
    const bool rotated = ROPE && d0 < p.rot;

    int64_t s, e;
    p.seq.find(n0, s, e);
    float ring[W > 1 ? W - 1 : 1][VEC];  // ring[i] = x[n-1-i]
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
    for (int64_t n = n0; n < n1; ++n) {
        if (n >= e) {
            p.seq.find(n, s, e);
            if (n == s) {  // a new sequence: nothing before it
#pragma unroll
                for (int i = 0; i < W - 1; ++i)
#pragma unroll
                    for (int c = 0; c < VEC; ++c) ring[i][c] = 0.f;
            }
        }
        float xv[VEC], acc[VEC];
        Vec16<E>::load(x + n * p.D, xv);
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            uint32_t ws[WS::kWords];
            WS::template load<WA>(w + (n * p.G + j[c]) * W, ws);
            float a = p.rho * xv[c];
#pragma unroll
            for (int k = 0; k < W; ++k) a = __builtin_fmaf(WS::at(ws, k), k == 0 ? xv[c] : ring[k - 1][c], a);
            acc[c] = a;
        }
        if constexpr (ROPE) {
            if (rotated) {
                float cs[VEC];
                load_turn<VEC>(p.rope + (int64_t)(n - s) * p.hd + (int32_t)(d0 % p.hd), cs);
                turn<VEC, false>(acc, cs);
            }
        }
        Vec16<E>::store(y + n * p.D, acc);
#pragma unroll
        for (int i = W - 2; i > 0; --i)
#pragma unroll
            for (int c = 0; c < VEC; ++c) ring[i][c] = ring[i - 1][c];
        if constexpr (W > 1) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) ring[0][c] = xv[c];
        }
    }
}

// dy of token t (a chunk of VEC channels), turned back at position pos when rotated.
template <class E, bool ROPE>
__device__ __forceinline__ void load_ds(const AnyParams &p, const typename E::store_t *g, int64_t t, int64_t pos,
                                        int64_t d0, bool rotated, float (&v)[E::kVec]) {
    constexpr int VEC = E::kVec;
    Vec16<E>::load(g + t * p.D, v);
    if constexpr (ROPE) {
        if (rotated) {
            float cs[VEC];
            load_turn<VEC>(p.rope + pos * p.hd + (int32_t)(d0 % p.hd), cs);
            turn<VEC, true>(v, cs);
        }
    }
}

template <class E, int W, bool ROPE>
__global__ __launch_bounds__(kAnyBlock) void hw_any_dx(AnyParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    const int64_t item = (int64_t)blockIdx.x * kAnyBlock + threadIdx.x;
    if (item >= p.items) return;
    const int64_t tile = item / p.nchunks;
    const int64_t chunk = item - tile * p.nchunks;
    const int64_t n0 = tile * kAnyTT;
    const int64_t n1 = min(n0 + (int64_t)kAnyTT, p.N);
    const int64_t d0 = chunk * VEC;
    const S *g = static_cast<const S *>(p.dy) + d0;
    const S *w = static_cast<const S *>(p.w);
    S *dx = static_cast<S *>(p.dx) + d0;
    int64_t j[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) j[c] = (d0 + c) / p.H;
    const bool rotated = ROPE && d0 < p.rot;

    int64_t s, e;
    p.seq.find(n0, s, e);
    for (int64_t m = n0; m < n1; ++m) {
        if (m >= e) p.seq.find(m, s, e);
        float acc[VEC];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const int64_t t = m + k;
            if (t >= e) break;  // m+k lies outside m's sequence (and every later tap too)
            float gt[VEC];
            load_ds<E, ROPE>(p, g, t, t - s, d0, rotated, gt);
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                const float wk = elem<E>(w, (t * p.G + j[c]) * W + k);
                if (k == 0) acc[c] = (wk + p.rho) * gt[c];
                else acc[c] = __builtin_fmaf(wk, gt[c], acc[c]);
            }
        }
        Vec16<E>::store(dx + m * p.D, acc);
    }
}

template <class E, int W, bool ROPE>
__global__ __launch_bounds__(kAnyBlock) void hw_any_dw(AnyParams p) {
    using S = typename E::store_t;
    constexpr int WA = pow2_align(W * (int)sizeof(S));
    const int64_t item = (int64_t)blockIdx.x * kAnyBlock + threadIdx.x;
    // every lane takes part in the butterfly below (segments of P lanes never
    // straddle a wave: P divides 64); lanes past the last segment add zeros
    const int64_t nseg = p.N * p.G;
    const int64_t seg0 = item / p.P;
    const int li = (int)(item - seg0 * p.P);
    const bool valid = seg0 < nseg;
    const int64_t seg = valid ? seg0 : nseg - 1;
    const int64_t n = seg / p.G;
    const int64_t jg = seg - n * p.G;
    const S *x = static_cast<const S *>(p.x);
    const S *g = static_cast<const S *>(p.dy);
    int64_t s, e;
    p.seq.find(n, s, e);
    const int64_t nv = n - s;  // taps k <= nv lie inside the sequence
    const int64_t pos = n - s;

    float part[W];
#pragma unroll
    for (int k = 0; k < W; ++k) part[k] = 0.f;
    if (valid) {
        for (int64_t dd = li; dd < p.H; dd += p.P) {
            const int64_t d = jg * p.H + dd;
            float gv = elem<E>(g, n * p.D + d);
            if constexpr (ROPE) {
                if (d < p.rot) {  // ds of channel d from its pair (2i, 2i+1)
                    const float go = elem<E>(g, n * p.D + (d ^ 1));
                    const float *cs = p.rope + (pos * (p.hd / 2) + (d % p.hd) / 2) * 2;
                    const float cv = cs[0], sv = cs[1];
                    gv = (d & 1) ? cv * gv - sv * go : cv * gv + sv * go;
                }
            }
#pragma unroll
            for (int k = 0; k < W; ++k)
                if (k <= nv) part[k] = __builtin_fmaf(gv, elem<E>(x, (n - k) * p.D + d), part[k]);
        }
    }
    for (int off = 1; off < p.P; off <<= 1)
#pragma unroll
        for (int k = 0; k < W; ++k) part[k] += __shfl_xor(part[k], off, kWave);
    if (valid && li == 0) Span<E, W>::template store<WA>(static_cast<S *>(p.dw) + seg * W, part);
}

template <class E>
AnyParams make_any(const HwProblem &pr) {
    AnyParams p;
    p.x = pr.x; p.w = pr.w; p.dy = pr.dy;
    p.y = pr.y; p.dx = pr.dx; p.dw = pr.dw;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N; p.D = pr.D; p.G = pr.D / pr.H;
    p.H = pr.H;
    p.rho = pr.residual ? 1.f : 0.f;
    p.nchunks = pr.D / E::kVec;
    p.items = (pr.N + kAnyTT - 1) / kAnyTT * p.nchunks;
    p.rope = pr.rope;
    p.rot = (int32_t)pr.rot;
    p.hd = pr.hd;
    p.npos = (int32_t)pr.max_pos;
    int lanes = 1;
    while (lanes < pr.H && lanes < kWave) lanes *= 2;
    p.P = lanes;
    return p;
}

int64_t blocks_of(int64_t items) { return (items + kAnyBlock - 1) / kAnyBlock; }

template <class E, int W, bool ROPE>
hipError_t launch_any(const HwProblem &pr, hipStream_t st, bool bwd) {
    const AnyParams p = make_any<E>(pr);
    if (p.N == 0) return hipSuccess;
    if (!bwd) {
        hipLaunchKernelGGL((hw_any_fwd<E, W, ROPE>), dim3((unsigned)blocks_of(p.items)), dim3(kAnyBlock), 0, st, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((hw_any_dx<E, W, ROPE>), dim3((unsigned)blocks_of(p.items)), dim3(kAnyBlock), 0, st, p);
    hipLaunchKernelGGL((hw_any_dw<E, W, ROPE>), dim3((unsigned)blocks_of(p.N * p.G * p.P)), dim3(kAnyBlock), 0, st,
                       p);
    return hipGetLastError();
}

template <class E, bool ROPE>
hipError_t dispatch_any(const HwProblem &pr, hipStream_t st, bool bwd) {
    switch (pr.W) {
        case 1: return launch_any<E, 1, ROPE>(pr, st, bwd);
        case 2: return launch_any<E, 2, ROPE>(pr, st, bwd);
        case 3: return launch_any<E, 3, ROPE>(pr, st, bwd);
        case 4: return launch_any<E, 4, ROPE>(pr, st, bwd);
        case 5: return launch_any<E, 5, ROPE>(pr, st, bwd);
        case 6: return launch_any<E, 6, ROPE>(pr, st, bwd);
        case 7: return launch_any<E, 7, ROPE>(pr, st, bwd);
        case 8: return launch_any<E, 8, ROPE>(pr, st, bwd);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t headwise_any(const HwProblem &p, hipStream_t s, bool bwd, bool rope) {
    if (p.dtype == Dtype::BF16)
        return rope ? dispatch_any<BF16, true>(p, s, bwd) : dispatch_any<BF16, false>(p, s, bwd);
    return rope ? dispatch_any<F32, true>(p, s, bwd) : dispatch_any<F32, false>(p, s, bwd);
}

}  // namespace dsc
