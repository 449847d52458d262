// decode.hip -- the dynamic short convolution at inference, one new token per
// sequence, with a rolling state of each sequence's last W-1 inputs, for
// gfx950.  The authors note that inference needs engineering of its own
// (gist.science technical summary, Significado y Reivindicaciones); the step
// is the forward of the same definitions (Methodology) evaluated at the
// sequence's newest token:
//   y[b,d] = rho*x[b,d] + w(b)_{d,0} x[b,d] + sum_{k=1}^{W-1} w(b)_{d,k} state[b,k-1,d]
//   state'[b,0,d] = x[b,d],  state'[b,i,d] = state[b,i-1,d]  (i >= 1)
// with w(b)_{d,k} = w[b, d/H, k] (head-wise) or sum_r z[b,r] U[r, d*W+k]
// (low rank, formed on chip).  state[b,i,d] holds the input of token t-1-i
// of sequence b, zero before its first token; a prefill hands its last W-1
// inputs over with dsc_state_from_prefill.
//
// Design: decoding moves a few MB per step, so launch latency and the number
// of dependent memory round trips bound it, not bandwidth.
//   * one thread per (sequence, 16-byte channel chunk): x, the state slots and
//     the filter are loaded once, y and the shifted state stored once (the
//     thread owns those state addresses, so the update is in place);
//   * low rank: a thread takes a few channels (16 bytes of U per rank) of one
//     sequence, lanes on consecutive sequences, so a wave's loads of U hit the
//     same addresses and the R-term sums (tens of MFLOP per step, on the
//     vector ALU) spread over about one wave per SIMD.  With so few waves the
//     kernel is latency-bound; the arrangements measured are listed in the
//     design notes.
#include "dsc_kernels.h"

namespace dsc {
namespace {

constexpr int kBlock = 256;

struct DecParams {
    const void *x, *w, *z, *U;
    void *state, *y;
    int64_t B, D, G;
    int32_t H, R;
    float rho;
    int64_t nchunks;
    // rotary embedding of y (head-wise + rotation only): channels [0, rot) in
    // heads of hd, table (npos, hd/2, 2), position pos[b] of sequence b's token
    const float *rope;
    const int32_t *pos;
    int32_t rot, hd, npos;
};

template <int VEC, int GPT>
__device__ __forceinline__ constexpr int grp(int c) {
    return GPT > 1 ? c / (VEC / GPT) : 0;
}

// y for one (sequence, chunk) from the input, the state slots and the
// per-channel taps (tap 0 already includes rho), turned by cs when ROT and
// rotated; then the state shift.
template <class E, int W, bool ROT = false>
__device__ __forceinline__ void finish(const float (&xv)[E::kVec], const float (&wt)[E::kVec][W],
                                       typename E::store_t *st, int64_t D, typename E::store_t *y,
                                       bool rotated = false, const float (&cs)[E::kVec] = {}) {
    constexpr int VEC = E::kVec;
    float sv[W > 1 ? W - 1 : 1][VEC];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) Vec16<E>::load(st + i * D, sv[i]);
    float acc[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
        float a = wt[c][0] * xv[c];
#pragma unroll
        for (int k = 1; k < W; ++k) a = __builtin_fmaf(wt[c][k], sv[k - 1][c], a);
        acc[c] = a;
    }
    if constexpr (ROT) {
        if (rotated) turn<VEC, false>(acc, cs);
    }
    Vec16<E>::store(y, acc);
    if constexpr (W > 1) {
#pragma unroll
        for (int i = W - 2; i > 0; --i) Vec16<E>::store(st + i * D, sv[i - 1]);
        Vec16<E>::store(st, xv);
    }
}

// Head-wise: thread = (sequence b, chunk), sequence fastest inside a chunk.
// ROPE: y of the first rot channels is then rotated at position pos[b]
// (a table row read once); a position outside [0, npos) has no row, and the
// sequence's rotated channels are set to NaN instead.
// GPT = 0 serves any H: each channel reads the filter of its own group d/H.
template <class E, int W, int GPT, bool ROPE>
__global__ __launch_bounds__(kBlock) void hw_decode_kernel(DecParams p) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int NW = (GPT > 0 ? GPT : 1) * W;
    constexpr int WALIGN = pow2_align(NW * (int)sizeof(S));
    // 32-bit index arithmetic: the API limits a decoding batch to B*D < 2^31
    const uint32_t B = (uint32_t)p.B;
    const uint32_t item = blockIdx.x * kBlock + threadIdx.x;
    if (item >= B * (uint32_t)p.nchunks) return;
    const uint32_t chunk = item / B;
    const int64_t b = item - chunk * B;
    const int64_t d0 = (int64_t)chunk * VEC;
    const int64_t jfirst = GPT > 1 ? (int64_t)chunk * GPT : d0 / p.H;

    float xv[VEC];
    Vec16<E>::load(static_cast<const S *>(p.x) + b * p.D + d0, xv);
    float wt[VEC][W];
    if constexpr (GPT == 0) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            float wf[W];
            Span<E, W>::template load<WALIGN>(static_cast<const S *>(p.w) + (b * p.G + (d0 + c) / p.H) * W, wf);
#pragma unroll
            for (int k = 0; k < W; ++k) wt[c][k] = wf[k] + (k == 0 ? p.rho : 0.f);
        }
    } else {
        float wf[NW];
        Span<E, NW>::template load<WALIGN>(static_cast<const S *>(p.w) + (b * p.G + jfirst) * W, wf);
#pragma unroll
        for (int c = 0; c < VEC; ++c)
#pragma unroll
            for (int k = 0; k < W; ++k) wt[c][k] = wf[grp<VEC, GPT>(c) * W + k] + (k == 0 ? p.rho : 0.f);
    }
    S *st = W > 1 ? static_cast<S *>(p.state) + b * (W - 1) * p.D + d0 : nullptr;  // no state when W = 1
    float cs[VEC];
    const bool rotated = ROPE && d0 < p.rot;
    if constexpr (ROPE) {
        if (rotated) {
            const int32_t m = p.pos[b];
            if (m >= 0 && m < p.npos) {
                load_turn<VEC>(p.rope + m * p.hd + (int32_t)d0 % p.hd, cs);
            } else {
#pragma unroll
                for (int c = 0; c < VEC; ++c) cs[c] = __builtin_nanf("");
            }
        }
    }
    finish<E, W, ROPE>(xv, wt, st, p.D, static_cast<S *>(p.y) + b * p.D + d0, rotated, cs);
}

// Channels per low-rank decoding thread: one 16-byte run of U per rank
// (CPT channels x W taps), a power of two.
template <class E, int W>
constexpr int lr_cpt() {
    int c = 16 / (W * (int)sizeof(typename E::store_t));
    int p2 = 1;
    while (p2 * 2 <= c) p2 *= 2;
    return p2;
}

// Low rank: thread = (sequence b, CPT channels), sequence fastest, so a
// wave's loads of U hit the same addresses.  The taps are sum over r of
// z[b,r] times CPT*W contiguous elements of row r of U, in groups of RB rank
// rows whose loads are all issued before any is used; with ZVEC (R a
// multiple of the z vector) z moves 16 bytes at a time, otherwise element by
// element.  Rows past R read row R-1 with a zero coefficient.
template <class E, int W, bool ZVEC>
__global__ __launch_bounds__(kBlock) void lr_decode_kernel(DecParams p) {
    using S = typename E::store_t;
    constexpr int CPT = lr_cpt<E, W>();
    constexpr int NU = CPT * W;                       // U elements per rank row
    constexpr int UAL = pow2_align(NU * (int)sizeof(S));
    constexpr int XAL = pow2_align(CPT * (int)sizeof(S));
    constexpr int RB = 16 / (int)sizeof(S);           // rank rows per group = one 16-byte vector of z
    // 32-bit index arithmetic: the API limits a decoding batch to B*D < 2^31
    const uint32_t B = (uint32_t)p.B, R = (uint32_t)p.R;
    const uint32_t nch = (uint32_t)p.D / CPT;
    const uint32_t item = blockIdx.x * kBlock + threadIdx.x;
    if (item >= B * nch) return;
    const uint32_t ch = item / B;
    const int64_t b = item - ch * B;
    const int64_t c0 = (int64_t)ch * CPT;

    float wt[CPT][W];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int k = 0; k < W; ++k) wt[c][k] = 0.f;
    const S *zb = static_cast<const S *>(p.z) + b * R;
    const S *Ub = static_cast<const S *>(p.U) + c0 * W;
    const int64_t DW = p.D * W;
    for (uint32_t r0 = 0; r0 < R; r0 += RB) {
        float uv[RB][NU], zr[RB];
        if constexpr (ZVEC) {
            Vec16<E>::load(zb + r0, zr);
        } else {
#pragma unroll
            for (int j = 0; j < RB; ++j) zr[j] = r0 + j < R ? load_elem<E>(zb + r0 + j) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const uint32_t r = r0 + j < R ? r0 + j : R - 1;
            Span<E, NU>::template load<UAL>(Ub + r * DW, uv[j]);
        }
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
            for (int e = 0; e < NU; ++e) wt[e / W][e % W] = __builtin_fmaf(zr[j], uv[j][e], wt[e / W][e % W]);
    }

    const S *xb = static_cast<const S *>(p.x) + b * p.D + c0;
    S *st = W > 1 ? static_cast<S *>(p.state) + b * (W - 1) * p.D + c0 : nullptr;
    float xv[CPT], sv[W > 1 ? W - 1 : 1][CPT], acc[CPT];
    Span<E, CPT>::template load<XAL>(xb, xv);
#pragma unroll
    for (int i = 0; i < W - 1; ++i) Span<E, CPT>::template load<XAL>(st + i * p.D, sv[i]);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        float a = (wt[c][0] + p.rho) * xv[c];
#pragma unroll
        for (int k = 1; k < W; ++k) a = __builtin_fmaf(wt[c][k], sv[k - 1][c], a);
        acc[c] = a;
    }
    Span<E, CPT>::template store<XAL>(static_cast<S *>(p.y) + b * p.D + c0, acc);
    if constexpr (W > 1) {
#pragma unroll
        for (int i = W - 2; i > 0; --i) Span<E, CPT>::template store<XAL>(st + i * p.D, sv[i - 1]);
        Span<E, CPT>::template store<XAL>(st, xv);
    }
}

// State after a prefill: thread = (sequence, slot i, chunk); slot i takes the
// sequence's token end-1-i, or zeros when the sequence is shorter.
template <class E>
__global__ __launch_bounds__(kBlock) void state_gather_kernel(const typename E::store_t *x, SeqMap seq,
                                                              int64_t nseq, int32_t slots, int64_t D,
                                                              int64_t nchunks, typename E::store_t *state) {
    constexpr int VEC = E::kVec;
    const int64_t item = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (item >= nseq * slots * nchunks) return;
    const int64_t chunk = item % nchunks;
    const int64_t si = item / nchunks;  // sequence * slots + slot
    const int64_t sq = si / slots;
    const int i = (int)(si - sq * slots);
    int64_t lo, hi;
    if (seq.cu != nullptr) {
        lo = seq.cu[sq];
        hi = seq.cu[sq + 1];
    } else {
        lo = sq * seq.T;
        hi = lo + seq.T;
    }
    const int64_t t = hi - 1 - i;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t >= lo) v = *reinterpret_cast<const uint4 *>(x + t * D + chunk * VEC);
    *reinterpret_cast<uint4 *>(state + si * D + chunk * VEC) = v;
}

template <class E>
DecParams make_params(const DecProblem &pr) {
    DecParams p;
    p.x = pr.x; p.w = pr.w; p.z = pr.z; p.U = pr.U;
    p.state = pr.state; p.y = pr.y;
    p.B = pr.B; p.D = pr.D;
    p.H = pr.H; p.R = pr.R;
    p.G = pr.H > 0 ? pr.D / pr.H : 0;
    p.rho = pr.residual ? 1.f : 0.f;
    p.nchunks = pr.D / E::kVec;
    p.rope = pr.rope;
    p.pos = pr.pos;
    p.rot = (int32_t)pr.rot;
    p.hd = pr.hd;
    p.npos = (int32_t)pr.max_pos;
    return p;
}

int64_t grid(int64_t items) { return (items + kBlock - 1) / kBlock; }

template <class E, int W, bool ROPE>
hipError_t launch_hw(const DecParams &p, int32_t H, int64_t blocks, hipStream_t st) {
    constexpr int VEC = E::kVec;
    if (H >= VEC ? H % VEC != 0 : VEC % H != 0) {  // groups that do not align with 16-byte chunks
        hipLaunchKernelGGL((hw_decode_kernel<E, W, 0, ROPE>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
    } else if (H >= VEC) {
        hipLaunchKernelGGL((hw_decode_kernel<E, W, 1, ROPE>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
    } else {
        switch (VEC / H) {
            case 2:
                hipLaunchKernelGGL((hw_decode_kernel<E, W, 2, ROPE>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
                break;
            case 4:
                hipLaunchKernelGGL((hw_decode_kernel<E, W, 4, ROPE>), dim3((unsigned)blocks), dim3(kBlock), 0, st, p);
                break;
            case 8:
                if constexpr (VEC >= 8) {
                    hipLaunchKernelGGL((hw_decode_kernel<E, W, 8, ROPE>), dim3((unsigned)blocks), dim3(kBlock), 0,
                                       st, p);
                    break;
                }
                return hipErrorInvalidValue;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <class E, int W>
hipError_t launch_w(const DecProblem &pr, hipStream_t st) {
    const DecParams p = make_params<E>(pr);
    if (p.B == 0) return hipSuccess;
    constexpr int VEC = E::kVec;
    const int64_t blocks = grid(p.B * p.nchunks);
    if (pr.lowrank) {
        const int64_t lr_blocks = grid(p.B * (p.D / lr_cpt<E, W>()));
        if (p.R % (16 / (int)sizeof(typename E::store_t)) == 0)  // z rows split into whole 16-byte vectors
            hipLaunchKernelGGL((lr_decode_kernel<E, W, true>), dim3((unsigned)lr_blocks), dim3(kBlock), 0, st, p);
        else
            hipLaunchKernelGGL((lr_decode_kernel<E, W, false>), dim3((unsigned)lr_blocks), dim3(kBlock), 0, st, p);
    } else if (pr.rot > 0) {
        return launch_hw<E, W, true>(p, pr.H, blocks, st);
    } else {
        return launch_hw<E, W, false>(p, pr.H, blocks, st);
    }
    return hipGetLastError();
}

template <class E>
hipError_t dispatch(const DecProblem &pr, hipStream_t st) {
    switch (pr.W) {
        case 1: return launch_w<E, 1>(pr, st);
        case 2: return launch_w<E, 2>(pr, st);
        case 3: return launch_w<E, 3>(pr, st);
        case 4: return launch_w<E, 4>(pr, st);
        case 5: return launch_w<E, 5>(pr, st);
        case 6: return launch_w<E, 6>(pr, st);
        case 7: return launch_w<E, 7>(pr, st);
        case 8: return launch_w<E, 8>(pr, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t decode_step(const DecProblem &p, hipStream_t s) {
    return p.dtype == Dtype::BF16 ? dispatch<BF16>(p, s) : dispatch<F32>(p, s);
}

hipError_t state_from_prefill(Dtype dt, const void *x, const int32_t *cu, int32_t n_seqs, int64_t B, int64_t T,
                              int64_t D, int32_t W, void *state, hipStream_t s) {
    const int64_t nseq = cu ? n_seqs : B;
    const int32_t slots = W - 1;
    if (slots == 0 || nseq == 0) return hipSuccess;
    const SeqMap seq{cu, n_seqs, T};
    if (dt == Dtype::BF16) {
        const int64_t nchunks = D / BF16::kVec;
        const int64_t blocks = grid(nseq * slots * nchunks);
        hipLaunchKernelGGL(state_gather_kernel<BF16>, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                           static_cast<const uint16_t *>(x), seq, nseq, slots, D, nchunks,
                           static_cast<uint16_t *>(state));
    } else {
        const int64_t nchunks = D / F32::kVec;
        const int64_t blocks = grid(nseq * slots * nchunks);
        hipLaunchKernelGGL(state_gather_kernel<F32>, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                           static_cast<const float *>(x), seq, nseq, slots, D, nchunks,
                           static_cast<float *>(state));
    }
    return hipGetLastError();
}

}  // namespace dsc
