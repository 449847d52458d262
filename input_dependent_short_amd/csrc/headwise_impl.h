// headwise_impl.h -- the head-wise kernels and their launchers, shared by
// headwise.hip (the layer alone) and rope.hip (the layer followed by the
// rotary position embedding of the query and key channels).  Internal to
// libdsc.so; each including file instantiates one value of ROPE, so the two
// sets of kernels compile in parallel.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: mechanism, parametrization (2) head-wise
// tying, placement with residual):
//   y[n,d] = rho*x[n,d] + sum_{k<W, n-k in seq(n)} w[n, d/H, k] * x[n-k, d]
// Backward for L = <dy, y>:
//   dx[m,d]   = rho*dy[m,d] + sum_{k<W, m+k in seq(m)} w[m+k, d/H, k] * dy[m+k, d]
//   dw[n,j,k] = [n-k in seq(n)] * sum_{d in group j} dy[n,d] * x[n-k, d]
// With ROPE, channels d < rot of y are then turned pair by pair (2i, 2i+1 of
// each head of hd channels) by the angle pos(n) * theta_i, the rotary
// embedding of "RoFormer: Enhanced Transformer with Rotary Position
// Embedding" (Su et al., Section 3.4.2), pos(n) = n - start of n's sequence;
// the backward first turns dy back (the transpose), then runs as above.
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
//     followed by a DPP butterfly over the H/VEC lanes of the group;
//   * the forward keeps the next batch of loads in flight while computing;
//   * the rotation reads cos / sin from an fp32 table (position, pair); a
//     16-byte chunk lies inside one head, so a thread's pairs are consecutive
//     entries of one row.  Each thread reads row p0 (the position of its
//     tile's first token) once.  bf16: the pair of cos / sin then turns by one
//     step (row 1) per token, back to (1, 0) at a sequence start, with no
//     memory access per token (the rounding drift over a tile, under 2e-5,
//     is far below bf16 resolution).  fp32: a token at p0 + j also reads row
//     j (rows j < TT + W are shared by every tile and stay in the L1 cache)
//     and combines it with row p0 by angle addition (about 2 ulp); a
//     sequence that starts inside the tile counts j from its own start;
//   * fp32 accumulation, one round-to-nearest-even store per output.
#pragma once

#include "dsc_kernels.h"

namespace dsc {
namespace {


struct HwParams {
    const void *x, *w, *dy;
    void *y, *dx, *dw;
    SeqMap seq;
    int64_t N, D, G;
    int32_t H;
    // Backward lane groups: a filter group of H >= VEC channels spans L =
    // H / VEC chunks and takes `lanes` (L rounded up to a power of two)
    // consecutive lanes, of which the first L are active; with H < VEC a
    // chunk holds whole groups and L = lanes = 1.
    int32_t lanes, L;
    float rho;
    int64_t nchunks, items;
    int64_t slots;    // backward lanes per token tile: (nchunks / L) * lanes
    int64_t lblocks;  // logical workgroups of kBlock work items
    const float *rope;  // (npos, hd/2, 2) cos, sin; read only by the ROPE kernels
    int32_t rot, hd;    // rotated channels [0, rot), head size
    int32_t npos;       // table rows
};

constexpr int kBlock = 256;

// Group-local index of channel c of a chunk in the thread's filter span.
template <int VEC, int GPT>
__device__ __forceinline__ constexpr int grp(int c) {
    return GPT > 1 ? c / (VEC / GPT) : 0;
}

// Cache policy of the streams each thread reads or writes once (x, w and
// dy rows of its own tile; y, dx and dw): nontemporal.  The halo rows before
// a tile, which the neighbouring tile also reads, keep the default policy.
#ifndef DSC_HW_NT
#define DSC_HW_NT 13  // bits: 1 x loads, 2 filter loads, 4 y / dx stores, 8 dy loads, 16 dw stores
#endif
constexpr bool kNT = (DSC_HW_NT & 1) != 0;
constexpr bool kNTW = (DSC_HW_NT & 2) != 0;
constexpr bool kNTS = (DSC_HW_NT & 4) != 0;
constexpr bool kNTG = (DSC_HW_NT & 8) != 0;
constexpr bool kNTD = (DSC_HW_NT & 16) != 0;

// Raw 16-byte vector of activations, widened to fp32 when used.
template <class E, bool NT = false>
__device__ __forceinline__ uint4 load_raw(const typename E::store_t *p) {
    return ld_u4<NT>(p);
}

template <class E>
__device__ __forceinline__ float lane_elem(const uint4 &v, int c) {
    const uint32_t w = c < (E::kVec / 4) ? v.x : c < 2 * (E::kVec / 4) ? v.y : c < 3 * (E::kVec / 4) ? v.z : v.w;
    if constexpr (E::kVec == 4) {
        return __uint_as_float(w);
    } else {
        return (c & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

template <class E>
__device__ __forceinline__ void unpack(const uint4 &v, float (&f)[E::kVec]) {
#pragma unroll
    for (int c = 0; c < E::kVec; ++c) f[c] = lane_elem<E>(v, c);
}

// Sum over aligned groups of `lanes` consecutive lanes (a power of two <= 64);
// every lane of the group receives the total.  DPP inside 16-lane rows
// (quad permutes, half-row and row mirrors), cross-lane shuffles beyond.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
    int o;
    switch (ctrl_sel) {
        case 0: o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, true); break;   // xor 1
        case 1: o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, true); break;   // xor 2
        case 2: o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, true); break;  // half-row mirror
        default: o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, true); break; // row mirror
    }
    return v + __int_as_float(o);
}

template <int NW>
__device__ __forceinline__ void group_sum(float (&v)[NW], int lanes) {
    if (lanes >= 2) {
#pragma unroll
        for (int i = 0; i < NW; ++i) v[i] = dpp_add(v[i], 0);
    }
    if (lanes >= 4) {
#pragma unroll
        for (int i = 0; i < NW; ++i) v[i] = dpp_add(v[i], 1);
    }
    if (lanes >= 8) {
#pragma unroll
        for (int i = 0; i < NW; ++i) v[i] = dpp_add(v[i], 2);
    }
    if (lanes >= 16) {
#pragma unroll
        for (int i = 0; i < NW; ++i) v[i] = dpp_add(v[i], 3);
    }
    if (lanes >= 32) {
#pragma unroll
        for (int i = 0; i < NW; ++i) v[i] += __shfl_xor(v[i], 16, kWave);
    }
    if (lanes >= 64) {
#pragma unroll
        for (int i = 0; i < NW; ++i) v[i] += __shfl_xor(v[i], 32, kWave);
    }
}

// One work item (a 16-byte channel chunk of one token tile) of the forward.
template <class E, int W, int GPT, int TT, int U, bool ROPE>
__device__ __forceinline__ void hw_fwd_item(const HwParams &p, int64_t item) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int NW = GPT * W;
    constexpr int WALIGN = pow2_align(NW * (int)sizeof(S));

    const int64_t tile = item / p.nchunks;
    const int64_t chunk = item - tile * p.nchunks;
    const int64_t n0 = tile * TT;
    const int64_t n1 = min(n0 + (int64_t)TT, p.N);
    const int64_t d0 = chunk * VEC;
    const int64_t jfirst = GPT > 1 ? chunk * GPT : d0 / p.H;

    const S *x = static_cast<const S *>(p.x) + d0;
    const S *w = static_cast<const S *>(p.w) + jfirst * W;
    S *y = static_cast<S *>(p.y) + d0;
    // rotated chunks: this thread's pairs start at entry (d0 mod hd)/2 of a table row
    const bool rotated = ROPE && d0 < p.rot;
    const float *tab = ROPE ? p.rope + (int32_t)d0 % p.hd : nullptr;

    int64_t s, e;
    p.seq.find(n0, s, e);
    // bf16 (REC): an is the cos / sin of the next token, stp one step;
    // fp32: an is the cos / sin at the tile's first token
    constexpr bool REC = ROPE && VEC == 8;
    float an[VEC], stp[VEC];
    if constexpr (ROPE) {
        if (rotated) {
            load_turn<VEC>(tab + (int32_t)(n0 - s) * p.hd, an);
            if constexpr (REC) {
                if (p.npos > 1) load_turn<VEC>(tab + p.hd, stp);
                else set_identity<VEC>(stp);
            }
        }
    }

    // ring[i] holds x[n-1-i]
    float ring[W > 1 ? W - 1 : 1][VEC];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int64_t t = n0 - 1 - i;
        if (t >= s) {
            unpack<E>(load_raw<E>(x + t * p.D), ring[i]);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) ring[i][c] = 0.f;
        }
    }

    // two batches of U tokens in flight: compute one while the next loads
    // filters stay raw words until used: as fp32 the two batches' filters
    // held 16 more registers (W = 4), which cost a wave per SIMD
    using WS = RawSpan<E, NW>;
    constexpr int NWW = WS::kWords;
    uint4 xa[U], xb[U];
    uint32_t wa[U][NWW], wb[U][NWW];
    auto load_batch = [&](int64_t nb, uint4 (&xr)[U], uint32_t (&wr)[U][NWW]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = nb + u;
            if (n < n1) {
                xr[u] = load_raw<E, kNT>(x + n * p.D);
                WS::template load<WALIGN, kNTW>(w + n * p.G * W, wr[u]);
            }
        }
    };
    auto compute_batch = [&](int64_t nb, const uint4 (&xr)[U], const uint32_t (&wr)[U][NWW]) {
        // the batch's offset rows, all requested before the first is used;
        // bit u of later: token u's sequence starts after n0 (no anchor)
        float cs[U][VEC];
        uint32_t later = 0;
        if constexpr (ROPE && !REC) {
            if (rotated) {
                int64_t ts = s, te = e;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t n = nb + u;
                    if (n < n1) {
                        if (n >= te) p.seq.find(n, ts, te);
                        later |= (uint32_t)(ts > n0) << u;
                        load_turn<VEC>(tab + (int32_t)(n - max(ts, n0)) * p.hd, cs[u]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = nb + u;
            if (n < n1) {
                if (n >= e) p.seq.find(n, s, e);
                const int64_t nv = n - s;  // taps k <= nv lie inside the sequence
                float xv[VEC], acc[VEC];
                unpack<E>(xr[u], xv);
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = p.rho * xv[c];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const bool ok = k <= nv;
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        const float wk = ok ? WS::at(wr[u], grp<VEC, GPT>(c) * W + k) : 0.f;
                        const float xk = k == 0 ? xv[c] : ring[k - 1][c];
                        acc[c] = __builtin_fmaf(wk, xk, acc[c]);
                    }
                }
                if constexpr (REC) {
                    if (rotated) {
                        if (nv == 0) set_identity<VEC>(an);
                        turn<VEC, false>(acc, an);
                        compose<VEC>(an, stp);
                    }
                } else if constexpr (ROPE) {
                    if (rotated) {
                        if (!((later >> u) & 1u)) compose<VEC>(cs[u], an);
                        turn<VEC, false>(acc, cs[u]);
                    }
                }
                Vec16<E>::template store<kNTS>(y + n * p.D, acc);
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
    };

    load_batch(n0, xa, wa);
    for (int64_t nb = n0; nb < n1; nb += 2 * U) {
        if (nb + U < n1) load_batch(nb + U, xb, wb);
        compute_batch(nb, xa, wa);
        if (nb + U >= n1) break;
        if (nb + 2 * U < n1) load_batch(nb + 2 * U, xa, wa);
        compute_batch(nb + U, xb, wb);
    }
}

// Workgroups of kBlock threads walk the logical blocks lb = blockIdx.x,
// blockIdx.x + gridDim.x, ... (one each when the grid covers them all; a
// grid of one round of resident workgroups otherwise), logical blocks
// remapped so that neighbouring tiles run on the same XCD (the grid is a
// multiple of 8 workgroups when it walks).
template <class E, int W, int GPT, int TT, int U, bool ROPE>
__global__ __launch_bounds__(kBlock) void hw_fwd_kernel(HwParams p) {
    for (int64_t lb = blockIdx.x; lb < p.lblocks; lb += gridDim.x) {
        const int64_t item = xcd_block_id(lb, p.lblocks) * kBlock + threadIdx.x;
        if (item < p.items) hw_fwd_item<E, W, GPT, TT, U, ROPE>(p, item);
    }
}

// One work item of the backward.
template <class E, int W, int GPT, int TT, int U, bool ROPE>
__device__ __forceinline__ void hw_bwd_item(const HwParams &p, int64_t item) {
    using S = typename E::store_t;
    constexpr int VEC = E::kVec;
    constexpr int NW = GPT * W;
    constexpr int WALIGN = pow2_align(NW * (int)sizeof(S));
    constexpr int WIN = U + W - 1;  // look-ahead window of (dy, w)

    const int64_t tile = item / p.slots;
    const int64_t slot = item - tile * p.slots;
    // lane li of filter group gi; padding lanes (li >= L) repeat the group's
    // last chunk, store nothing and add zeros to the group sum
    const int64_t gi = slot / p.lanes;
    const int li = (int)(slot - gi * p.lanes);
    const bool active = li < p.L;
    const int64_t chunk = gi * p.L + (active ? li : p.L - 1);
    const int64_t n0 = tile * TT;
    const int64_t n1 = min(n0 + (int64_t)TT, p.N);
    const int64_t d0 = chunk * VEC;
    const int64_t jfirst = GPT > 1 ? chunk * GPT : d0 / p.H;
    const bool leader = li == 0;

    const S *x = static_cast<const S *>(p.x) + d0;
    const S *g = static_cast<const S *>(p.dy) + d0;
    const S *w = static_cast<const S *>(p.w) + jfirst * W;
    S *dx = static_cast<S *>(p.dx) + d0;
    S *dw = static_cast<S *>(p.dw) + jfirst * W;
    const bool rotated = ROPE && d0 < p.rot;
    const float *tab = ROPE ? p.rope + (int32_t)d0 % p.hd : nullptr;

    int64_t s, e;
    p.seq.find(n0, s, e);
    int64_t ls = s, le = e;  // sequence of the newest look-ahead token (ROPE)
    // as in the forward: bf16 (REC) turns an by stp per look-ahead token
    constexpr bool REC = ROPE && VEC == 8;
    float an[VEC], stp[VEC];
    if constexpr (ROPE) {
        if (rotated) {
            load_turn<VEC>(tab + (int32_t)(n0 - s) * p.hd, an);
            if constexpr (REC) {
                if (p.npos > 1) load_turn<VEC>(tab + p.hd, stp);
                else set_identity<VEC>(stp);
            }
        }
    }

    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    uint4 ring[W > 1 ? W - 1 : 1];  // ring[i] = x[m-1-i] (raw)
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
        const int64_t t = n0 - 1 - i;
        ring[i] = t >= s ? load_raw<E>(x + t * p.D) : zero4;
    }
    // look-ahead window: slot i holds token mb + i
    using WS = RawSpan<E, NW>;  // filters as raw words, widened where used
    constexpr int NWW = WS::kWords;
    uint4 gw[WIN];
    uint32_t ww[WIN][NWW];
    auto load_gw = [&](int64_t t, int slot) {
        if (t < p.N) {
            gw[slot] = load_raw<E, kNTG>(g + t * p.D);
            WS::template load<WALIGN, kNTW>(w + t * p.G * W, ww[slot]);
        } else {
            gw[slot] = zero4;
#pragma unroll
            for (int c = 0; c < NWW; ++c) ww[slot][c] = 0u;
        }
    };
    // ROPE: the window holds dy turned back, in fp32 (gf); cos / sin of a
    // token are requested with its dy and applied when the slot is first used.
    float gf[WIN][VEC];
    // Look-ahead token t in stream order.  REC: returns whether t starts a
    // sequence.  fp32: requests the offset row of t and returns whether t's
    // sequence starts after n0 (no anchor then).
    auto load_cs = [&](int64_t t, float (&cs)[VEC]) {
        bool flag = false;
        if (rotated && t < p.N) {
            if (t >= le) p.seq.find(t, ls, le);
            if constexpr (REC) {
                flag = t == ls;
            } else {
                flag = ls > n0;
                load_turn<VEC>(tab + (int32_t)(t - max(ls, n0)) * p.hd, cs);
            }
        }
        return flag;
    };
    // dy of token t turned back, into the fp32 window (slots settle in stream order)
    auto settle = [&](int64_t t, int slot, float (&cs)[VEC], bool flag) {
        unpack<E>(gw[slot], gf[slot]);
        if (rotated && t < p.N) {
            if constexpr (REC) {
                if (flag) set_identity<VEC>(an);
                turn<VEC, true>(gf[slot], an);
                compose<VEC>(an, stp);
            } else {
                if (!flag) compose<VEC>(cs, an);
                turn<VEC, true>(gf[slot], cs);
            }
        }
    };
#pragma unroll
    for (int i = 0; i < W - 1; ++i) load_gw(n0 + i, i);
    if constexpr (ROPE) {
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            float cs[VEC];
            const bool lat = load_cs(n0 + i, cs);
            settle(n0 + i, i, cs, lat);
        }
    }

    for (int64_t mb = n0; mb < n1; mb += U) {
        uint4 xv[U];
        float cs[U][VEC];
        uint32_t later = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t m = mb + u;
            xv[u] = m < n1 ? load_raw<E, kNT>(x + m * p.D) : zero4;
            load_gw(mb + W - 1 + u, W - 1 + u);
            if constexpr (ROPE) later |= (uint32_t)load_cs(mb + W - 1 + u, cs[u]) << u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t m = mb + u;
            if (m < n1) {
                if constexpr (ROPE) settle(mb + W - 1 + u, W - 1 + u, cs[u], (later >> u) & 1u);
                if (m >= e) p.seq.find(m, s, e);
                const int64_t ahead = e - m;  // dx terms k < ahead stay in the sequence
                const int64_t back = m - s;   // dw taps k <= back stay in the sequence
                float gm[VEC], acc[VEC];
                if constexpr (ROPE) {
#pragma unroll
                    for (int c = 0; c < VEC; ++c) gm[c] = gf[u][c];
                } else {
                    unpack<E>(gw[u], gm);
                }
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[c] = p.rho * gm[c];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const bool ok = k < ahead;
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        const float wk = ok ? WS::at(ww[u + k], grp<VEC, GPT>(c) * W + k) : 0.f;
                        float gk;
                        if constexpr (ROPE) gk = gf[u + k][c];
                        else gk = k == 0 ? gm[c] : lane_elem<E>(gw[u + k], c);
                        acc[c] = __builtin_fmaf(wk, gk, acc[c]);
                    }
                }
                if (active) Vec16<E>::template store<kNTS>(dx + m * p.D, acc);

                float part[NW];
#pragma unroll
                for (int i = 0; i < NW; ++i) part[i] = 0.f;
                // bf16 with filter groups of whole channel pairs: the dw partials are
                // 2-term dot products of the packed dy and x words (fp32 sums, no
                // widening); otherwise fp32 multiply-adds of the widened values
                constexpr bool DOT = VEC == 8 && GPT <= 4 && !ROPE;
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const uint4 &xr = k == 0 ? xv[u] : ring[k - 1];
                    if constexpr (DOT) {
                        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                        const uint32_t xw[4] = {xr.x, xr.y, xr.z, xr.w};
                        const uint32_t gd[4] = {gw[u].x, gw[u].y, gw[u].z, gw[u].w};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            part[grp<VEC, GPT>(2 * j) * W + k] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf2, gd[j]), __builtin_bit_cast(bf2, xw[j]),
                                part[grp<VEC, GPT>(2 * j) * W + k], false);
                    } else {
#pragma unroll
                        for (int c = 0; c < VEC; ++c)
                            part[grp<VEC, GPT>(c) * W + k] =
                                __builtin_fmaf(gm[c], lane_elem<E>(xr, c), part[grp<VEC, GPT>(c) * W + k]);
                    }
                }
                if (!active) {
#pragma unroll
                    for (int i = 0; i < NW; ++i) part[i] = 0.f;
                }
                group_sum<NW>(part, p.lanes);
#pragma unroll
                for (int q = 0; q < GPT; ++q)
#pragma unroll
                    for (int k = 0; k < W; ++k)
                        if (k > back) part[q * W + k] = 0.f;
                if (leader) Span<E, NW>::template store<WALIGN, kNTD>(dw + m * p.G * W, part);

#pragma unroll
                for (int i = W - 2; i > 0; --i) ring[i] = ring[i - 1];
                if constexpr (W > 1) ring[0] = xv[u];
            }
        }
        // slide the look-ahead window by U tokens
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            if constexpr (ROPE) {
#pragma unroll
                for (int c = 0; c < VEC; ++c) gf[i][c] = gf[U + i][c];
            } else {
                gw[i] = gw[U + i];
            }
#pragma unroll
            for (int c = 0; c < NWW; ++c) ww[i][c] = ww[U + i][c];
        }
    }
}

template <class E, int W, int GPT, int TT, int U, bool ROPE>
__global__ __launch_bounds__(kBlock) void hw_bwd_kernel(HwParams p) {
    for (int64_t lb = blockIdx.x; lb < p.lblocks; lb += gridDim.x) {
        const int64_t item = xcd_block_id(lb, p.lblocks) * kBlock + threadIdx.x;
        // Whole filter groups are in or out of range together (items is a
        // multiple of slots, which is a multiple of lanes), so skipping here
        // never strands a lane that a group reduction reads.
        if (item < p.items) hw_bwd_item<E, W, GPT, TT, U, ROPE>(p, item);
    }
}

#ifndef DSC_HW_TT
#define DSC_HW_TT 32
#endif
#ifndef DSC_HW_U
#define DSC_HW_U 4
#endif
constexpr int kTT = DSC_HW_TT;  // tokens per thread tile
constexpr int kU = DSC_HW_U;    // tokens per load batch

template <class E>
HwParams make_params(const HwProblem &pr, int64_t tt, bool bwd, int64_t &blocks) {
    HwParams p;
    p.x = pr.x; p.w = pr.w; p.dy = pr.dy;
    p.y = pr.y; p.dx = pr.dx; p.dw = pr.dw;
    p.seq = SeqMap{pr.cu, pr.n_seqs, pr.T};
    p.N = pr.N; p.D = pr.D; p.G = pr.D / pr.H;
    p.H = pr.H;
    p.L = pr.H >= E::kVec ? pr.H / E::kVec : 1;
    p.lanes = 1;
    while (p.lanes < p.L) p.lanes *= 2;
    p.rho = pr.residual ? 1.f : 0.f;
    p.nchunks = pr.D / E::kVec;
    p.slots = p.nchunks / p.L * p.lanes;
    p.rope = pr.rope;
    p.rot = (int32_t)pr.rot;
    p.hd = pr.hd;
    p.npos = (int32_t)pr.max_pos;
    const int64_t ntiles = (pr.N + tt - 1) / tt;
    p.items = ntiles * (bwd ? p.slots : p.nchunks);
    p.lblocks = (p.items + kBlock - 1) / kBlock;
    blocks = p.lblocks;
    return p;
}

// The backward takes tiles of 2*kTT tokens when those still give at least
// one whole round of resident waves (measured on MI355X: 7% faster at
// B=4 T=4096 D=8192, much slower when the grid no longer fills the chip).
#ifndef DSC_HW_PERSIST
#define DSC_HW_PERSIST 1
#endif
// Grid of a launch over `lblocks` logical workgroups: all of them, or (when
// they need more than one round of resident workgroups) one round, a
// multiple of 8, whose workgroups then walk the logical blocks.  One round
// avoids the ramp between rounds.
inline int64_t hw_grid(int64_t lblocks, int bpc) {
    if (!DSC_HW_PERSIST) return lblocks;
    int64_t round = (int64_t)device_cus() * bpc;
    round -= round % 8;
    return (round >= 8 && lblocks > round) ? round : lblocks;
}

template <class E, int W, int GPT, bool ROPE>
hipError_t launch_w(const HwProblem &pr, hipStream_t st, bool bwd) {
    constexpr int UB = kU;
    int64_t blocks;
    if (bwd) {
        static const int bpc = blocks_per_cu(
            reinterpret_cast<const void *>(&hw_bwd_kernel<E, W, GPT, 2 * kTT, UB, ROPE>), kBlock);
        HwParams p = make_params<E>(pr, 2 * kTT, true, blocks);
        const int64_t waves_long = p.items / kWave;
        if (waves_long >= (int64_t)device_cus() * bpc * (kBlock / kWave)) {
            if (blocks)
                hipLaunchKernelGGL((hw_bwd_kernel<E, W, GPT, 2 * kTT, UB, ROPE>), dim3((unsigned)hw_grid(blocks, bpc)),
                                   dim3(kBlock), 0, st, p);
            return hipGetLastError();
        }
        static const int bpc_short = blocks_per_cu(
            reinterpret_cast<const void *>(&hw_bwd_kernel<E, W, GPT, kTT, UB, ROPE>), kBlock);
        p = make_params<E>(pr, kTT, true, blocks);
        if (blocks)
            hipLaunchKernelGGL((hw_bwd_kernel<E, W, GPT, kTT, UB, ROPE>), dim3((unsigned)hw_grid(blocks, bpc_short)),
                               dim3(kBlock), 0, st, p);
        return hipGetLastError();
    }
    static const int bpc_fwd = blocks_per_cu(
        reinterpret_cast<const void *>(&hw_fwd_kernel<E, W, GPT, kTT, kU, ROPE>), kBlock);
    HwParams p = make_params<E>(pr, kTT, false, blocks);
    if (blocks)
        hipLaunchKernelGGL((hw_fwd_kernel<E, W, GPT, kTT, kU, ROPE>), dim3((unsigned)hw_grid(blocks, bpc_fwd)),
                           dim3(kBlock), 0, st, p);
    return hipGetLastError();
}

template <class E, int GPT, bool ROPE>
hipError_t dispatch_w(const HwProblem &pr, hipStream_t st, bool bwd) {
    switch (pr.W) {
        case 1: return launch_w<E, 1, GPT, ROPE>(pr, st, bwd);
        case 2: return launch_w<E, 2, GPT, ROPE>(pr, st, bwd);
        case 3: return launch_w<E, 3, GPT, ROPE>(pr, st, bwd);
        case 4: return launch_w<E, 4, GPT, ROPE>(pr, st, bwd);
        case 5: return launch_w<E, 5, GPT, ROPE>(pr, st, bwd);
        case 6: return launch_w<E, 6, GPT, ROPE>(pr, st, bwd);
        case 7: return launch_w<E, 7, GPT, ROPE>(pr, st, bwd);
        case 8: return launch_w<E, 8, GPT, ROPE>(pr, st, bwd);
        default: return hipErrorInvalidValue;
    }
}

template <class E, bool ROPE>
hipError_t dispatch(const HwProblem &pr, hipStream_t st, bool bwd) {
    constexpr int VEC = E::kVec;
    if (pr.H >= VEC) return dispatch_w<E, 1, ROPE>(pr, st, bwd);
    switch (VEC / pr.H) {
        case 2: return dispatch_w<E, 2, ROPE>(pr, st, bwd);
        case 4: return dispatch_w<E, 4, ROPE>(pr, st, bwd);
        case 8:
            if constexpr (VEC >= 8) return dispatch_w<E, 8, ROPE>(pr, st, bwd);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace dsc
