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
#include <algorithm>

#include "dsc_common.h"
#include "dsc_kernels.h"

namespace dsc {
namespace {


// Groups per tile: BN = TG*W columns of w (a multiple of 16 for any W <= 8).
constexpr int gen_tg(int W) { return W <= 4 ? 32 : 16; }
// Token rows per tile of the fused kernels (4 waves).  Tiles of 256 rows on
// 8 waves (one block per CU, 6 stages) measured slower, for the fused and the
// plain products alike (MLP ~2B, K = 2048: forward 323 against 277 us,
// backward 931 against 815 us), so every kernel takes 128 rows.
constexpr int gen_bm(int) { return 128; }
constexpr int gen_threads(int W) { return 2 * gen_bm(W); }  // 64 threads per 32 rows

// ------------------------------------------- matrix-core GEMM, direct loads
//
// The products whose operands are both K-contiguous (the generator h V^T and
// dh = dw V^T... with V transposed) run a four-stage pipeline: each stage is
// a kDBK = 32 slice of K, loaded by buffer_load ... lds straight from memory
// into LDS (no registers), three stages ahead of the matrix cores.  A stage
// holds the A tile (BM rows) then the B tile (BN <= 128 rows), rows of 64
// bytes whose four 16-byte chunks are placed at chunk ^ chunk_swz(row), chunk_swz(r) =
// ((r >> 1) ^ (r >> 2)) & 3, so that the 16 rows a fragment read touches fall
// on distinct banks whether the LDS serves 16 lanes over 64 banks or 8 lanes
// over 32 banks per cycle (measured: the plain (r >> 2) placement left four
// conflict cycles per LDS instruction cycle).  Each
// stage is an LDS array of its own, so the compiler can tell which load a
// fragment read waits for; a stage is refilled only after a barrier that all
// waves pass once they are done reading it.  Out-of-range rows lie past the
// buffer resource and out-of-range k take the offset kFar: both read as zero.

constexpr int kDBK = 32;
__device__ __forceinline__ int chunk_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
typedef __attribute__((address_space(3))) void lds_void;

template <int BR, int NW>
constexpr int dma_per_wave() {
    return (BR / 16 + NW - 1) / NW;
}

// Tile configuration: BM rows of A by BN rows of B (the columns of C) on
// BM / 32 waves (4 or 8), NST stages of kStage bytes (A tile, then B tile);
// the fp32 result tile is parked RPS rows per stage.  WM x WN waves, each
// MF x NF fragments of 16 x 16.  The 256-row tiles (8 waves, 6 stages) keep
// about 1.7 times the bytes of the 128-row ones in flight per CU and load a
// quarter fewer operand bytes per product.
template <int BM, int BN>
struct DCfg {
    static constexpr int NW = BM / 32;
    static constexpr int kThreads = 64 * NW;
    static constexpr int NST = BM == 256 ? 6 : 4;
    static constexpr int kA = BM * 64, kB = BN * 64;
    static constexpr int kStage = BM == 256 ? 24576 : 16384;
    static constexpr int RPS = 32;  // result rows per stage (a shift in the epilogues)
    static constexpr int WN = (BN / 2) % 16 == 0 ? 2 : 1, WM = NW / WN;
    static constexpr int MF = BM / WM / 16, NF = BN / WN / 16;
    static constexpr int kPerTile = dma_per_wave<BM, NW>() + dma_per_wave<BN, NW>();
    static_assert(kA + kB <= kStage && RPS * BN * 4 <= kStage && 4 * RPS >= BM && MF >= 1 && NF >= 1,
                  "tile configuration");
};

// The stage arrays of a block (NST of them used).
struct Stages {
    unsigned char *s[6];
};

// Direct loads of one operand tile (BR rows, kDBK k from k0) into dst.  A
// wave instruction fills 64 consecutive 16-byte slots; the BR/16 of them are
// spread over the NW waves, and a wave with no instruction left repeats the
// last one (same bytes to the same place), so every wave issues the same
// count per tile.
template <int BR, int NW>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int64_t ld, int64_t k0, int64_t K,
                                         unsigned char *dst, int wave, int lane) {
    constexpr int kInst = BR / 16, kPer = dma_per_wave<BR, NW>();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = wave + NW * j < kInst ? wave + NW * j : kInst - 1;
        const int slot = 64 * i + lane;
        const int row = slot >> 2, logical = (slot & 3) ^ chunk_swz(row);
        const int64_t kk = k0 + 8 * logical;
        // k past K: bit 31 set, past every tile's resource (a tile spans < 2^31 bytes); arithmetic rather
        // than a select, which the compiler would turn into a branch around the load
        const uint32_t off = (uint32_t)(((int64_t)row * ld + kk) * 2) | ((uint32_t)(kk >= K) << 31);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + 1024 * i), 16, off, 0, 0, 0);
    }
}

// C[BM x BN] = A[m0 .., :] . B[n0 .., :]^T (both K-contiguous, K % 8 == 0),
// fp32: acc[mf][nf][j] = C[RM*wm + 16mf + 4(lane>>4) + j][RN*wn + 16nf + (lane&15)]
// with RM = BM/WM, RN = BN/WN, (wm, wn) = (wave / WN, wave % WN).  Ends with
// every load landed and a barrier: the stages may then be reused.
template <int BM, int BN>
__device__ __forceinline__ void dma_gemm(const uint16_t *A, int64_t lda, int64_t M, const uint16_t *B, int64_t ldb,
                                         int64_t Nc, int64_t K, int64_t m0, int64_t n0, const Stages &S,
                                         floatx4 (&acc)[DCfg<BM, BN>::MF][DCfg<BM, BN>::NF]) {
    using C = DCfg<BM, BN>;
    constexpr int NST = C::NST;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t mr = min((int64_t)BM, M - m0), nr = min((int64_t)BN, Nc - n0);
    const __amdgpu_buffer_rsrc_t ra = make_stream(A + m0 * lda, mr > 0 ? mr * lda * 2 : 0);
    const __amdgpu_buffer_rsrc_t rb = make_stream(B + n0 * ldb, nr > 0 ? nr * ldb * 2 : 0);
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < C::NF; ++nf) acc[mf][nf] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto issue = [&](int64_t t, unsigned char *st) {
        dma_tile<BM, C::NW>(ra, lda, t * kDBK, K, st, wave, lane);
        dma_tile<BN, C::NW>(rb, ldb, t * kDBK, K, st + C::kA, wave, lane);
    };
    // fragment rows: A rows RM*wm + 16mf + (lane&15), B rows RN*wn + 16nf + (lane&15); chunk lane>>4
    const int c = lane >> 4;
    int aoff[C::MF], boff[C::NF];
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf) {
        const int r = (BM / C::WM) * wm + 16 * mf + (lane & 15);
        aoff[mf] = r * 64 + 16 * (c ^ chunk_swz(r));
    }
#pragma unroll
    for (int nf = 0; nf < C::NF; ++nf) {
        const int r = (BN / C::WN) * wn + 16 * nf + (lane & 15);
        boff[nf] = C::kA + r * 64 + 16 * (c ^ chunk_swz(r));
    }
    auto compute = [&](const unsigned char *st) {
        bf16x8 a[C::MF], b[C::NF];
#pragma unroll
        for (int mf = 0; mf < C::MF; ++mf) a[mf] = *reinterpret_cast<const bf16x8 *>(st + aoff[mf]);
#pragma unroll
        for (int nf = 0; nf < C::NF; ++nf) b[nf] = *reinterpret_cast<const bf16x8 *>(st + boff[nf]);
#pragma unroll
        for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
            for (int nf = 0; nf < C::NF; ++nf)
                acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mf], b[nf], acc[mf][nf], 0, 0, 0);
    };
    // tile t waits until only the loads of tiles t+1 .. t+NST-2 are in flight,
    // then a barrier makes every wave's loads of tile t visible (and ends every
    // wave's reads of the stage that tile t+NST-1 refills)
    auto step = [&](int64_t t, unsigned char *cur, unsigned char *refill) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * C::kPerTile) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(t + NST - 1, refill);
        compute(cur);
    };
    const int64_t nk = (K + kDBK - 1) / kDBK;
#pragma unroll
    for (int j = 0; j < NST - 1; ++j) issue(j, S.s[j]);
    // whole rounds of NST tiles: tiles past nk read as zero and add nothing
    for (int64_t t = 0; t < nk; t += NST) {
#pragma unroll
        for (int j = 0; j < NST; ++j) step(t + j, S.s[j], S.s[(j + NST - 1) % NST]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// The fp32 result tile of dma_gemm parked in the first four stages: row r
// in stage r / 32 at (r % 32) * bn floats.  The stage is picked by selects
// (an array indexed by r would be kept in memory, LDS or scratch, per thread).
struct CsView {
    unsigned char *s0, *s1, *s2, *s3;
    int bn;
    __device__ __forceinline__ float *wrow(int r) const {
        unsigned char *b = r < 64 ? (r < 32 ? s0 : s1) : (r < 96 ? s2 : s3);
        return reinterpret_cast<float *>(b) + (r & 31) * bn;
    }
    __device__ __forceinline__ const float *row(int r) const { return wrow(r); }
};

template <int BM, int BN>
__device__ __forceinline__ void dma_park(const floatx4 (&acc)[DCfg<BM, BN>::MF][DCfg<BM, BN>::NF], const CsView &cs) {
    using C = DCfg<BM, BN>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
    for (int mf = 0; mf < C::MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < C::NF; ++nf)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cs.wrow((BM / C::WM) * wm + 16 * mf + 4 * (lane >> 4) + j)[(BN / C::WN) * wn + 16 * nf + (lane & 15)] =
                    acc[mf][nf][j];
}

// Element by element: an aggregate initializer made only of LDS addresses
// would be emitted as a constant in global memory, which cannot hold them.
__device__ __forceinline__ void set_stages(Stages &S, CsView &cs, unsigned char *a, unsigned char *b,
                                           unsigned char *c, unsigned char *d, unsigned char *e, unsigned char *f,
                                           int bn) {
    S.s[0] = cs.s0 = a;
    S.s[1] = cs.s1 = b;
    S.s[2] = cs.s2 = c;
    S.s[3] = cs.s3 = d;
    S.s[4] = e;
    S.s[5] = f;
    cs.bn = bn;
}

// The stage arrays of a kernel with tile configuration C (NST of them sized).
#define DSC_GEN_STAGES(C)                                                                         \
    __shared__ __align__(16) unsigned char st0[C::kStage], st1[C::kStage], st2[C::kStage],      \
        st3[C::kStage], st4[C::NST > 4 ? C::kStage : 16], st5[C::NST > 5 ? C::kStage : 16];      \
    Stages S;                                                                                      \
    CsView cs;                                                                                     \
    set_stages(S, cs, st0, st1, st2, st3, st4, st5, C::kB / 64)

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

constexpr int kSeg = 16;  // tokens one thread walks in the epilogues

// Row n of x (clamped into [0, N)) as raw bf16 bits, 8 channels from c.
__device__ __forceinline__ uint4 row8(const uint16_t *base, int64_t n, int64_t N, int64_t D, int64_t c) {
    const int64_t r = n < 0 ? 0 : (n >= N ? N - 1 : n);
    return *reinterpret_cast<const uint4 *>(base + r * D + c);
}

__device__ __forceinline__ float elem8(const uint4 &v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// y of tokens n0 + t0 .. + kSeg - 1 (those below N) for channels c .. c+7.
// UNI: the 8 channels share one group (H % 8 == 0): one filter read per tap.
template <int W, bool UNI>
__device__ __forceinline__ void fwd_walk(const GenParams &p, const CsView &cs, const int64_t *seq_start,
                                         int64_t n0, int t0, int64_t c, int64_t g0) {
    constexpr int NR = kSeg + W - 1;
    uint4 xr[NR];  // rows n0 + t0 - (W-1) + i
#pragma unroll
    for (int i = 0; i < NR; ++i) xr[i] = row8(p.x, n0 + t0 - (W - 1) + i, p.N, p.D, c);
    int col[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) col[e] = (int)((c + (UNI ? 0 : e)) / p.H - g0) * W;
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
        const int t = t0 + j;
        const int64_t n = n0 + t;
        if (n >= p.N) break;
        const int64_t s = seq_start[t];
        const float *wrow = cs.row(t);
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = p.rho * elem8(xr[j + W - 1], e);
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const bool in = n - k >= s;
            if constexpr (UNI) {
                const float wk = in ? wrow[col[0] + k] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(wk, elem8(xr[j + W - 1 - k], e), out[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    out[e] = __builtin_fmaf(in ? wrow[col[e] + k] : 0.f, elem8(xr[j + W - 1 - k], e), out[e]);
            }
        }
        store8(p.y + n * p.D + c, out);
    }
}

// Forward: block = (token tile, group tile), walked so that the group tiles
// of one token tile (which share its rows of h) run on one XCD.
template <int W>
__global__ __launch_bounds__(gen_threads(W), 512 / gen_threads(W))
void gen_fwd_kernel(GenParams p) {
    constexpr int TG = gen_tg(W), BN = TG * W, BM = gen_bm(W);
    using C = DCfg<BM, BN>;
    static_assert(C::kThreads == gen_threads(W), "block size");
    DSC_GEN_STAGES(C);
    __shared__ int64_t seq_start[BM];
    const int64_t lb = xcd_block_id(blockIdx.x, (int64_t)gridDim.x);
    const int64_t tn = lb / p.ntiles_g, tg = lb - tn * p.ntiles_g;
    const int64_t n0 = tn * BM, g0 = tg * TG;
    const int tid = threadIdx.x;
    if (tid < BM && n0 + tid < p.N) {
        int64_t s, e;
        p.seq.find(n0 + tid, s, e);
        seq_start[tid] = s;
    }
    floatx4 acc[C::MF][C::NF];
    dma_gemm<BM, BN>(p.h, p.K, p.N, p.V, p.K, p.G * W, p.K, n0, g0 * W, S, acc);
    dma_park<BM, BN>(acc, cs);
    __syncthreads();

    // y of the tile's tokens over the channels of groups [g0, g0 + gcount):
    // a thread walks kSeg consecutive tokens of one 8-channel chunk, with the
    // kSeg + W - 1 rows of x it reads loaded up front (no load depends on a
    // branch); consecutive threads take consecutive chunks of the same rows
    const int64_t gcount = min((int64_t)TG, p.G - g0);
    const int64_t c0 = g0 * p.H;
    const int nchunks = (int)(gcount * p.H / 8);
    const bool uniform = p.H % 8 == 0;  // a chunk's 8 channels share one group
    for (int it = tid; it < nchunks * (BM / kSeg); it += C::kThreads) {
        const int sg = it / nchunks, q = it - sg * nchunks;
        if (n0 + kSeg * sg >= p.N) break;  // items are in segment order
        if (uniform) fwd_walk<W, true>(p, cs, seq_start, n0, kSeg * sg, c0 + 8 * q, g0);
        else fwd_walk<W, false>(p, cs, seq_start, n0, kSeg * sg, c0 + 8 * q, g0);
    }
}

// dx and dw of tokens n0 + t0 .. + kSeg - 1 (those below N and inside the
// tile's kStep outputs) for channels c .. c+7 of group g (column gl of the
// tile), H % 8 == 0.  The group's cpg = H/8 chunks sit on cpg consecutive
// lanes (a power of two, aligned), which sum dw with butterfly shuffles; the
// first of them stores it.  All rows are loaded before they are used.
template <int W>
__device__ __forceinline__ void bwd_walk(const GenParams &p, const CsView &cs, const int64_t *seq_start,
                                         const int64_t *seq_end, int64_t n0, int t0, int kStep, int64_t c, int gl,
                                         int64_t g, int cpg, bool lead) {
    constexpr int NR = kSeg + W - 1;
    const int64_t N = p.N, D = p.D;
    uint4 gr[NR];  // dy rows n0 + t0 + i
#pragma unroll
    for (int i = 0; i < NR; ++i) gr[i] = row8(p.dy, n0 + t0 + i, N, D, c);
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
        const int t = t0 + j;
        const int64_t m = n0 + t;
        if (t >= kStep || m >= N) break;
        const int64_t e_ = seq_end[t];
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = p.rho * elem8(gr[j], e);
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const float wk = m + k < e_ ? cs.row(t + k)[gl * W + k] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(wk, elem8(gr[j + k], e), out[e]);
        }
        store8(p.dx + m * D + c, out);
    }
    uint4 xr[NR];  // x rows n0 + t0 - (W-1) + i
#pragma unroll
    for (int i = 0; i < NR; ++i) xr[i] = row8(p.x, n0 + t0 - (W - 1) + i, N, D, c);
    const int64_t GW = p.G * W;
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
        const int t = t0 + j;
        const int64_t m = n0 + t;
        if (t >= kStep || m >= N) break;
        const int64_t s_ = seq_start[t];
        float dws[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            float v = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) v = __builtin_fmaf(elem8(gr[j], e), elem8(xr[j + W - 1 - k], e), v);
            dws[k] = m - k >= s_ ? v : 0.f;
        }
        for (int off = 1; off < cpg; off <<= 1)
#pragma unroll
            for (int k = 0; k < W; ++k) dws[k] += __shfl_xor(dws[k], off);
        if (lead) {
            uint16_t *dst = p.dw + m * GW + g * W;
#pragma unroll
            for (int k = 0; k < W; ++k) dst[k] = to_bf16(dws[k]);
        }
    }
}

// Backward, w recomputed: tile rows [n0, n0 + BM) with n0 = tile * kStep;
// dx and dw of tokens [n0, n0 + kStep).  MODE 2 (H % 8 == 0, H/8 a power of
// two up to 64): segment walks per 8-channel chunk (bwd_walk).  Otherwise one
// (token, group) per item, so a group's filter gradient is summed in
// registers, with 8 channels per load (MODE 1, H % 8 == 0) or one (MODE 0).
template <int W, int MODE>
__global__ __launch_bounds__(gen_threads(W), 512 / gen_threads(W))
void gen_bwd_kernel(GenParams p) {
    constexpr int TG = gen_tg(W), BN = TG * W, BM = gen_bm(W);
    using C = DCfg<BM, BN>;
    constexpr int kStep = BM - (W - 1);
    DSC_GEN_STAGES(C);
    __shared__ int64_t seq_start[BM], seq_end[BM];
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
    floatx4 acc[C::MF][C::NF];
    dma_gemm<BM, BN>(p.h, p.K, p.N, p.V, p.K, p.G * W, p.K, n0, g0 * W, S, acc);
    dma_park<BM, BN>(acc, cs);
    __syncthreads();

    const int gcount = (int)min((int64_t)TG, p.G - g0);
    const int64_t D = p.D, GW = p.G * W;
    const int H = p.H;
    if constexpr (MODE == 2) {
        const int cpg = H / 8, nchunks = gcount * cpg;
        for (int it = tid; it < nchunks * (BM / kSeg); it += C::kThreads) {
            const int sg = it / nchunks, q = it - sg * nchunks;
            if (kSeg * sg >= kStep || n0 + kSeg * sg >= p.N) break;  // items are in segment order
            const int gl = q / cpg;
            bwd_walk<W>(p, cs, seq_start, seq_end, n0, kSeg * sg, kStep, g0 * H + 8 * q, gl, g0 + gl, cpg,
                        (q & (cpg - 1)) == 0);
        }
        return;
    }
    constexpr int VEC = MODE == 1 ? 8 : 1;
    for (int it = tid; it < kStep * gcount; it += C::kThreads) {
        const int t = it / gcount, gl = it - t * gcount;
        const int64_t m = n0 + t;
        if (m >= p.N) break;
        const int64_t s = seq_start[t], e = seq_end[t];
        // taps whose token stays in m's sequence: dx reads m+k (k < ahead), dw reads m-k (k < back)
        const int ahead = (int)min((int64_t)W, e - m), back = (int)min((int64_t)W, m - s + 1);
        float wk[W];
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k] = k < ahead ? cs.row(t + k)[gl * W + k] : 0.f;
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

// Plain product C (M x Nc) = A . B^T (both K-contiguous) over k in
// [ks * kc, min(K, (ks + 1) * kc)) for split ks = blockIdx / tiles, stored as
// OUT at C + ks * split_stride (the partial sums of a split-K product, or
// the product itself with one split).
constexpr int kPBM = 128, kPBN = 128;  // tile of the plain products
using PlainCfg = DCfg<kPBM, kPBN>;

template <class OUT>
__global__ __launch_bounds__(PlainCfg::kThreads, 2) void dma_gemm_kernel(const uint16_t *A, int64_t lda,
                                                                         const uint16_t *B, int64_t ldb, int64_t M,
                                                                         int64_t Nc, int64_t K, int64_t kc, OUT *C,
                                                                         int64_t ldc, int64_t split_stride,
                                                                         int64_t ntiles_n, int64_t ntiles) {
    constexpr int BM = kPBM, BN = kPBN;
    using L = PlainCfg;
    DSC_GEN_STAGES(L);
    (void)cs;
    const int64_t lb = xcd_block_id(blockIdx.x, (int64_t)gridDim.x);
    const int64_t ks = lb / ntiles, tile = lb - ks * ntiles;
    const int64_t tm = tile / ntiles_n, tn = tile - tm * ntiles_n;
    const int64_t m0 = tm * BM, n0 = tn * BN, kb = ks * kc;
    floatx4 acc[L::MF][L::NF];
    dma_gemm<BM, BN>(A + kb, lda, M, B + kb, ldb, Nc, min(kc, K - kb), m0, n0, S, acc);
    OUT *Cs = C + ks * split_stride;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / L::WN, wn = wave % L::WN;
#pragma unroll
    for (int mf = 0; mf < L::MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < L::NF; ++nf) {
            const int64_t col = n0 + (BN / L::WN) * wn + 16 * nf + (lane & 15);
            if (col >= Nc) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = m0 + (BM / L::WM) * wm + 16 * mf + 4 * (lane >> 4) + j;
                if (row >= M) continue;
                if constexpr (sizeof(OUT) == 4) Cs[row * ldc + col] = acc[mf][nf][j];
                else Cs[row * ldc + col] = to_bf16(acc[mf][nf][j]);
            }
        }
}

// dst[c][r] = src[r][c] for r < rows, 0 for rows <= r < ldd (src rows x cols,
// dst cols x ldd; cols and ldd multiples of 4).  64 x 64 tiles through LDS,
// 8-byte accesses.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *src, int64_t rows, int64_t cols,
                                                        uint16_t *dst, int64_t ldd) {
    __shared__ uint16_t tile[64][68];
    const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + ty + 16 * i, c = c0 + 4 * tx;
        uint2 v = make_uint2(0u, 0u);
        if (r < rows && c < cols) v = *reinterpret_cast<const uint2 *>(src + r * cols + c);
        tile[ty + 16 * i][4 * tx] = (uint16_t)(v.x & 0xffffu);
        tile[ty + 16 * i][4 * tx + 1] = (uint16_t)(v.x >> 16);
        tile[ty + 16 * i][4 * tx + 2] = (uint16_t)(v.y & 0xffffu);
        tile[ty + 16 * i][4 * tx + 3] = (uint16_t)(v.y >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + ty + 16 * i, r = r0 + 4 * tx;
        if (c >= cols || r >= ldd) continue;
        const int cl = ty + 16 * i;
        const uint2 v = make_uint2((uint32_t)tile[4 * tx][cl] | ((uint32_t)tile[4 * tx + 1][cl] << 16),
                                   (uint32_t)tile[4 * tx + 2][cl] | ((uint32_t)tile[4 * tx + 3][cl] << 16));
        *reinterpret_cast<uint2 *>(dst + c * ldd + r) = v;
    }
}

hipError_t transpose(const uint16_t *src, int64_t rows, int64_t cols, uint16_t *dst, int64_t ldd, hipStream_t st) {
    const dim3 grid((unsigned)((ldd + 63) / 64), (unsigned)((cols + 63) / 64));
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, rows, cols, dst, ldd);
    return hipGetLastError();
}

// dst[i] = sum over s < nparts of src[s * n + i], in order of s.
__global__ __launch_bounds__(256) void sum_splits(const float *src, int64_t nparts, int64_t n, float *dst) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = 0.f;
    for (int64_t s = 0; s < nparts; ++s) acc += src[s * n + i];
    dst[i] = acc;
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
    constexpr int TG = gen_tg(W), BM = gen_bm(W);
    const int64_t G = pr.D / pr.H;
    const int64_t tn = (pr.N + BM - 1) / BM, tg = (G + TG - 1) / TG;
    const GenParams p = make_gen(pr, tn, tg);
    hipLaunchKernelGGL((gen_fwd_kernel<W>), dim3((unsigned)(tn * tg)), dim3(DCfg<BM, TG * W>::kThreads), 0, st, p);
    return hipGetLastError();
}

// The backward's workspace: dw (N x GW), V^T (K x GW), dw^T (GW x Np), h^T
// (K x Np) in bf16, with Np = N rounded up to 32 (zero columns past N), and
// the fp32 partial sums of dV when its K = Np reduction is split.
struct GenBwdPlan {
    int64_t GW, Np, splits, kc;
    size_t off_vt, off_dwt, off_ht, off_parts, bytes;
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

GenBwdPlan gen_bwd_plan(int64_t N, int64_t D, int32_t W, int32_t H, int64_t K) {
    GenBwdPlan pl;
    pl.GW = (D / H) * W;
    pl.Np = (N + 31) / 32 * 32;
    // dV has ceil(GW/128) * ceil(K/128) output tiles; split its token sum
    // until about 512 blocks run (splits of at least 1024 tokens, at most 32)
    const int64_t tiles = ((pl.GW + 127) / 128) * ((K + 127) / 128);
    int64_t sp = tiles < 512 ? (512 + tiles - 1) / tiles : 1;
    sp = std::min<int64_t>(std::min<int64_t>(sp, 32), std::max<int64_t>(1, pl.Np / 1024));
    pl.kc = ((pl.Np + sp - 1) / sp + 31) / 32 * 32;
    pl.splits = (pl.Np + pl.kc - 1) / pl.kc;
    size_t o = align256((size_t)N * pl.GW * 2);
    pl.off_vt = o;
    o += align256((size_t)K * pl.GW * 2);
    pl.off_dwt = o;
    o += align256((size_t)pl.GW * pl.Np * 2);
    pl.off_ht = o;
    o += align256((size_t)K * pl.Np * 2);
    pl.off_parts = o;
    if (pl.splits > 1) o += align256((size_t)pl.splits * pl.GW * K * 4);
    pl.bytes = o;
    return pl;
}

template <int W>
hipError_t gen_bwd_w(const GenProblem &pr, hipStream_t st) {
    constexpr int TG = gen_tg(W), BM = gen_bm(W);
    constexpr int kStep = BM - (W - 1);
    constexpr int kThr = DCfg<BM, TG * W>::kThreads;
    const int64_t G = pr.D / pr.H, GW = G * W;
    const int64_t tn = (pr.N + kStep - 1) / kStep, tg = (G + TG - 1) / TG;
    const GenBwdPlan pl = gen_bwd_plan(pr.N, pr.D, pr.W, pr.H, pr.K);
    unsigned char *ws = static_cast<unsigned char *>(pr.dw);
    uint16_t *Vt = reinterpret_cast<uint16_t *>(ws + pl.off_vt);
    uint16_t *dwT = reinterpret_cast<uint16_t *>(ws + pl.off_dwt);
    uint16_t *hT = reinterpret_cast<uint16_t *>(ws + pl.off_ht);
    float *parts = reinterpret_cast<float *>(ws + pl.off_parts);
    const GenParams p = make_gen(pr, tn, tg);
    const int cpg = pr.H / 8;
    if (pr.H % 8 == 0 && cpg <= 64 && (cpg & (cpg - 1)) == 0)
        hipLaunchKernelGGL((gen_bwd_kernel<W, 2>), dim3((unsigned)(tn * tg)), dim3(kThr), 0, st, p);
    else if (pr.H % 8 == 0)
        hipLaunchKernelGGL((gen_bwd_kernel<W, 1>), dim3((unsigned)(tn * tg)), dim3(kThr), 0, st, p);
    else
        hipLaunchKernelGGL((gen_bwd_kernel<W, 0>), dim3((unsigned)(tn * tg)), dim3(kThr), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dh (N x K) = dw (N x GW) . (V^T)^T, both with GW contiguous
    if ((e = transpose(p.V, GW, pr.K, Vt, GW, st)) != hipSuccess) return e;
    {
        const int64_t tm = (pr.N + kPBM - 1) / kPBM, tk = (pr.K + kPBN - 1) / kPBN;
        hipLaunchKernelGGL((dma_gemm_kernel<uint16_t>), dim3((unsigned)(tm * tk)), dim3(PlainCfg::kThreads), 0, st, p.dw, GW, Vt,
                           GW, pr.N, pr.K, GW, GW, static_cast<uint16_t *>(pr.dh), pr.K, (int64_t)0, tk, tm * tk);
    }
    // dV (GW x K) = dw^T . (h^T)^T over the Np (zero-padded) tokens, in splits
    // of kc tokens summed in order afterwards
    if ((e = transpose(p.dw, pr.N, GW, dwT, pl.Np, st)) != hipSuccess) return e;
    if ((e = transpose(p.h, pr.N, pr.K, hT, pl.Np, st)) != hipSuccess) return e;
    {
        const int64_t tm = (GW + kPBM - 1) / kPBM, tk = (pr.K + kPBN - 1) / kPBN;
        float *out = pl.splits > 1 ? parts : pr.dV;
        hipLaunchKernelGGL((dma_gemm_kernel<float>), dim3((unsigned)(tm * tk * pl.splits)), dim3(PlainCfg::kThreads), 0, st, dwT,
                           pl.Np, hT, pl.Np, GW, pr.K, pl.Np, pl.kc, out, pr.K, GW * pr.K, tk, tm * tk);
        if (pl.splits > 1)
            hipLaunchKernelGGL(sum_splits, dim3((unsigned)((GW * pr.K + 255) / 256)), dim3(256), 0, st, parts,
                               pl.splits, GW * pr.K, pr.dV);
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

hipError_t generate_filters(const uint16_t *h, const uint16_t *V, int64_t N, int64_t K, int64_t C, uint16_t *w,
                            hipStream_t st) {
    const int64_t tm = (N + kPBM - 1) / kPBM, tc = (C + kPBN - 1) / kPBN;
    hipLaunchKernelGGL((dma_gemm_kernel<uint16_t>), dim3((unsigned)(tm * tc)), dim3(PlainCfg::kThreads), 0, st, h, K, V, K, N, C,
                       K, K, w, C, (int64_t)0, tc, tm * tc);
    return hipGetLastError();
}

size_t headwise_gen_bwd_workspace(int64_t N, int64_t D, int32_t W, int32_t H, int64_t K) {
    return gen_bwd_plan(N, D, W, H, K).bytes;
}

hipError_t headwise_gen_fwd(const GenProblem &p, hipStream_t s) { DSC_GEN_W_SWITCH(p.W, gen_fwd_w<Wc>(p, s)); }

hipError_t headwise_gen_bwd(const GenProblem &p, hipStream_t s) { DSC_GEN_W_SWITCH(p.W, gen_bwd_w<Wc>(p, s)); }

}  // namespace dsc
