// lowrank_taps.hip -- backward of the fused low-rank convolution for ranks
// 33..64 and W = 2..4 (bf16), with the taps of every 32-channel slice split
// over two waves, for gfx950.
//
// Operation ("Dynamic Short Convolutions Improve Transformers", gist.science
// technical summary, Methodology: mechanism; parametrization (1), the
// low-rank factorisation w(t) = z_t U; the backward is the chain rule of the
// mechanism for L = <dy, y>):
//   w[n,d,k]    = sum_r z[n,r] U[r, d*W+k]
//   dx[m,d]     = rho dy[m,d] + sum_k [m in seq(m+k)] w[m+k,d,k] dy[m+k,d]
//   dwc[n,d,k]  = [n-k in seq(n)] dy[n,d] x[n-k,d]            (rounded to bf16)
//   dz[n,r]     = sum_{d,k} U[r, d*W+k] dwc[n,d,k]
//   dU[r,d*W+k] = sum_n z[n,r] dwc[n,d,k]
//
// Design.  A block of 8 waves owns 4 slices of 32 channels and a token range
// walked in 16-token steps.  The two waves of a slice split it by channels:
// wave HF takes channels 4HF .. 4HF+3 of every 8-channel chunk, for dx, dwc,
// dz and dU alike, and loads only those 8 bytes of each x and dy row (the
// two waves together read each row once).  Each wave keeps the U operands of
// its 16 channels (both matrix-core layouts) and their dU tiles, half of what
// one wave doing the whole slice needs, so that two waves fit per SIMD and
// one wave's matrix-core products overlap the other's vector work.  Per step
// a wave forms
//   * dwc of every tap (x shifted back by k): by pairs of taps the B operand
//     of dz^T += U dwc, and staged as dwc^T in LDS for dU;
//   * w of every tap for tokens n+k on the matrix cores (U_k^T z, the z rows
//     read from one LDS ring shared by the block) and dx with dy shifted ahead
//     by k (DPP row moves, filled from the next step), written as bf16 into
//     the pair's dx tile in LDS.
// The x refill is issued between the two parts and the dy refill after them,
// so each load is in flight while half a step runs.  Per 32-token pair the
// block meets two barriers (LDS only: loads and stores in flight stay in
// flight).  At the next pair's start all threads store the pair's dx tile as
// whole rows of the block's 128 channels (two tiles, pairs alternate).
// Between the barriers every wave adds the pair's dU on the matrix cores
// (operands re-read transposed from LDS), and the dz partials of the 8 waves
// are summed in LDS in a fixed order and added to an fp32 accumulator with
// one atomic per (token, rank).  The z ring (8 slots of 16 rows and a copy of
// slot 0, so that every step's rows and the W-1 after them are contiguous)
// is written two pairs ahead by all threads of the block.  dU stays in
// registers over the whole range and is added with coalesced atomics at the
// end, as in the one-wave-per-slice kernel of lowrank.hip.
#include "lowrank_common.h"

namespace dsc {
namespace {

constexpr int kTapWaves = 8;
constexpr int kTapThreads = kTapWaves * kWave;
// Register rings of x and dy, in steps (each load is in flight for about half
// a step with 2 slots; with 4 slots for either, the walk unrolls 4 steps and
// the W = 4 instances spill inside the loop).  The walk unrolls kTapRing
// steps, a multiple of both depths and of the 2-step pair.
#ifndef DSC_TAP_RING_X
#define DSC_TAP_RING_X 2
#endif
#ifndef DSC_TAP_RING_G
#define DSC_TAP_RING_G 2
#endif
constexpr int kTapRingX = DSC_TAP_RING_X;
constexpr int kTapRingG = DSC_TAP_RING_G;
constexpr int kTapRing = kTapRingX > kTapRingG ? kTapRingX : kTapRingG;
static_assert(kTapRing % kTapRingX == 0 && kTapRing % kTapRingG == 0 && kTapRing % 2 == 0, "ring depths");

template <int V> struct HalfTag { static constexpr int value = V; };

template <int W>
struct TapLds {
    static constexpr int KP = (W + 1) / 2;  // pairs of taps (the K groups of dz's products)
    static constexpr int RP = 64;           // padded rank
    static constexpr int PZ = 2 * RP + 8;   // bytes per z row
    static constexpr int kZ = 9 * 16 * PZ;  // 8 slots of 16 rows + a copy of slot 0
    static constexpr int PW = 40;           // bytes per token row of dwc^T (the wave's 16 channels + pad)
    static constexpr int kDwcWave = W * 32 * PW;
    static constexpr int PD = 4 * RP + 16;  // bytes per token row of dz partials
    static constexpr int kDzWave = 32 * PD;
    static constexpr int oDwc = kZ;
    static constexpr int oDz = oDwc + kTapWaves * kDwcWave;
    static constexpr int oDxt = oDz + kTapWaves * kDzWave;
    static constexpr int kDxt = 32 * 256;        // a pair's dx rows of the block's 128 channels (bf16)
    static constexpr int kLoop = oDxt + 2 * kDxt;  // two tiles: pairs alternate
    static constexpr int kDuPitch = 32 * W + 1;  // floats per rank row of a slice's staged dU tile
    static constexpr int kDuSlice = RP * kDuPitch * 4;
    static constexpr int kBytes = kLoop > 4 * kDuSlice ? kLoop : 4 * kDuSlice;
    static_assert(kBytes + kTapWaves * 4 * kSeqWords <= 160 * 1024, "the block must fit the LDS of a CU");
};

// ZV: R % 4 == 0, z rows move as 8-byte vectors.  ROPE: the layer is followed
// by the rotary embedding of channels [0, p.rot) (heads of p.hd), so dy is
// turned back at each token's position before use: each step's dy as it is
// first read (the dx part of the step before), with its cos, sin from the
// table loaded at that step's start.
template <int W, bool ZV, bool ROPE>
__global__ __launch_bounds__(kTapThreads, 1) void lr_bwd_taps(LrParams p, int64_t nslices, int64_t tpb) {
    using L = TapLds<W>;
    constexpr int P = kTapRing;    // steps per unrolled walk iteration
    constexpr int PX = kTapRingX;  // x ring slots
    constexpr int PG = kTapRingG;  // dy ring slots
    constexpr int RT = 4;  // 16-row rank tiles
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];
    __shared__ uint32_t seq_words[kTapWaves][kSeqWords];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = wid & 3;
    const int half = wid >> 2;
    const int64_t ngroups = (nslices + 3) / 4;
    const int64_t tchunk = blockIdx.x / ngroups;
    const int64_t group = blockIdx.x - tchunk * ngroups;
    const int64_t d0 = (group * 4 + slice) * 32;
    const int64_t nbeg = tchunk * tpb;
    const int64_t nend = min(nbeg + tpb, p.N);
    const int64_t nsteps = ((nend - nbeg + 16 * P - 1) / (16 * P)) * P;  // whole rings

    const int tok = lane & 15;
    const int q = lane >> 4;
    const int i16 = lane & 15;
    // the wave's 4 channels of the lane's 8-channel chunk: the two waves of a
    // slice take its channels 4*half .. 4*half+3 of every chunk
    const int64_t cbase = d0 + 8 * q + 4 * half;
    const bool chan_ok = cbase < p.D;
    const int R = p.R;
    const int64_t N = p.N;
    const int64_t D = p.D;
    const int64_t DW = D * W;

    const uint16_t *xg = static_cast<const uint16_t *>(p.x);
    const uint16_t *gg = static_cast<const uint16_t *>(p.dy);
    const uint16_t *zg = static_cast<const uint16_t *>(p.z);
    const uint16_t *U = static_cast<const uint16_t *>(p.U);
    uint16_t *dxg = static_cast<uint16_t *>(p.dx);

    unsigned char *zring = lds;
    unsigned char *dwcT = lds + L::oDwc + wid * L::kDwcWave;  // [tap][32 tokens][PW]
    unsigned char *dzb = lds + L::oDz + wid * L::kDzWave;     // [32 tokens][PD]
    // dx of a pair, [32 tokens][16 chunks of 8 channels], chunk c of row r at
    // position c ^ (r & 15) (16 rows at one chunk hit distinct banks); pair p
    // writes tile p % 2 during its steps, and the block stores it at the start
    // of pair p + 1
    unsigned char *dxt = lds + L::oDxt;

    StartBits<kSeqWords> starts;
    starts.build(seq_words[wid], p.seq, N, nbeg - 32, lane);
    SeqPos sp{0};
    if constexpr (ROPE) {
        int64_t s_, e_;
        p.seq.find(nbeg < N ? nbeg : N - 1, s_, e_);
        sp.start = s_;
    }
    // dy of a step turned back by the rotation of its token's position (the
    // channel pairs (cbase, cbase+1) and (cbase+2, cbase+3); a group of 4 lies
    // wholly inside or outside [0, rot) since rot is a multiple of the head
    // size, itself a multiple of 8)
    const bool rope_lane = ROPE && chan_ok && cbase < p.rot;
    auto turn_back = [&](uint2 &v, const float (&cs)[4]) {
        if (rope_lane) {
            uint32_t w2[2] = {v.x, v.y};
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                const float a = bf16_lo(w2[i2]), b = bf16_hi(w2[i2]);
                const float c = cs[2 * i2], sn = cs[2 * i2 + 1];
                w2[i2] = pack_bf16x2(a * c + b * sn, b * c - a * sn);
            }
            v = make_uint2(w2[0], w2[1]);
        }
    };

    // ---- x, dy and dx streams of the wave's slice, as in lowrank.hip
    const uint32_t act_step = (uint32_t)(16 * D * 2);
    const uint32_t xoff = chan_ok ? (uint32_t)((tok * D + cbase) * 2) : kFar;
    const __amdgpu_buffer_rsrc_t rx = make_stream(xg + nbeg * D, (N - nbeg) * D * 2);
    const __amdgpu_buffer_rsrc_t rg = make_stream(gg + nbeg * D, (N - nbeg) * D * 2);
    const __amdgpu_buffer_rsrc_t rdx = make_stream(dxg + nbeg * D, (nend - nbeg) * D * 2);
    auto fetch_x = [&](int64_t step) { return buf_load8<kLrNtX>(rx, xoff + (uint32_t)step * act_step); };
    auto fetch_g = [&](int64_t step) { return buf_load8<kLrNtG>(rg, xoff + (uint32_t)step * act_step); };
    // the pair's dx tile to memory as whole rows of the block's 128 channels
    // (256 bytes, two cache lines): thread = row tid/16, position tid%16
    uint32_t dxt_off;
    {
        const int row = tid >> 4;
        const int64_t ch = group * 128 + 8 * ((tid & 15) ^ (row & 15));
        dxt_off = ch < D ? (uint32_t)((row * D + ch) * 2) : kFar;
    }
    auto store_dx = [&](int64_t first_step) {
        const uint4 v = *reinterpret_cast<const uint4 *>(dxt + ((first_step >> 1) & 1) * L::kDxt + 16 * tid);
        buf_store16<kLrNtDx>(rdx, dxt_off + (uint32_t)first_step * act_step, v);
    };

    // ---- z rows by pairs of steps (32 rows): thread = row tid/16, ranks 4*(tid%16) .. +3
    const int zrow = tid >> 4;
    const int zc = tid & 15;
    const uint32_t zpair = (uint32_t)(32 * R * 2);
    const __amdgpu_buffer_rsrc_t rz = make_stream(zg + nbeg * R, (N - nbeg) * R * 2);
    const uint32_t zoff = 4 * zc < R ? (uint32_t)((zrow * R + 4 * zc) * 2) : kFar;
    auto fetch_zp = [&](int64_t pair) -> uint2 {
        if constexpr (ZV) {
            return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rz, zoff + (uint32_t)pair * zpair, 0, 0));
        } else {
            const int64_t n = nbeg + 32 * pair + zrow;
            uint32_t h[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r0 = 4 * zc + 2 * e;
                const uint32_t lo = (n < N && r0 < R) ? zg[n * R + r0] : 0u;
                const uint32_t hi = (n < N && r0 + 1 < R) ? zg[n * R + r0 + 1] : 0u;
                h[e] = lo | (hi << 16);
            }
            return make_uint2(h[0], h[1]);
        }
    };
    // slot of step s = s mod 8; slot 0 is also written after slot 7
    auto write_zp = [&](int64_t pair, uint2 v) {
        const int slot = (int)((2 * pair + (zrow >> 4)) & 7);
        const int row = zrow & 15;
        *reinterpret_cast<uint2 *>(zring + (16 * slot + row) * L::PZ + 8 * zc) = v;
        if (slot == 0) *reinterpret_cast<uint2 *>(zring + (128 + row) * L::PZ + 8 * zc) = v;
    };
    write_zp(0, fetch_zp(0));
    write_zp(1, fetch_zp(1));
    uint2 zpf = fetch_zp(2);

    // ---- register rings: x step s in slot s % PX (read with slot s-1), dy
    // step s in slot s % PG (read with slot s+1)
    uint2 xr[PX], gr[PG];
#pragma unroll
    for (int j = 0; j < PX - 1; ++j) xr[j] = fetch_x(j);
    xr[PX - 1] = make_uint2(0u, 0u);  // step -1: only its last W-1 tokens are read
    {
        const int64_t n = nbeg - 16 + tok;
        if (n >= 0 && n < N && tok >= 16 - (W - 1) && chan_ok)
            xr[PX - 1] = *reinterpret_cast<const uint2 *>(xg + n * D + cbase);
    }
#pragma unroll
    for (int j = 0; j < PG; ++j) gr[j] = fetch_g(j);
    if constexpr (ROPE) {  // step 0's dy
        float cs[4];
        rope_cs<4>(p, sp.pos_and_advance(starts, nbeg, tok), cbase, cs);
        turn_back(gr[0], cs);
    }
    lds_barrier();  // the ring's first two pairs

    // dz atomics: this thread's rank (= lane) and tokens wid + 8*it of a pair
    const unsigned char *dz_all = lds + L::oDz;

    auto walk = [&](auto half_tag) {
        constexpr int HF = decltype(half_tag)::value;
        // U operands kept in registers for the whole walk (the wave's channels
        // d0 + 8c' + 4HF + j, j < 4, of every chunk c'):
        //   ua (dx): rows channel d0 + 8(i>>2) + 4HF + (i&3), K rank 32c + 8(lane>>4) + e
        //   ub (dz, taps 2kp and 2kp+1): rows rank 16rt + (lane&15), K element e of
        //     lane group q = lane>>4: channel d0 + 8q + 4HF + (e&3), tap 2kp + (e>>2)
        constexpr int KP = L::KP;
        bf16x8 ua[W][2];
        bf16x8 ub[KP][RT];
        {
            const int64_t ch = d0 + 8 * (i16 >> 2) + 4 * HF + (i16 & 3);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 32 * c + 8 * q + e;
                    uint16_t v[W];
                    const bool ok = r < R && ch < D;  // else read U's start, zeroed by the mask
                    const uint16_t m = (uint16_t)keep_mask(ok);
                    load_taps<W>(U + (ok ? ((int64_t)r * D + ch) * W : 0), v);
#pragma unroll
                    for (int k = 0; k < W; ++k) ua[k][c][e] = __builtin_bit_cast(__bf16, (uint16_t)(v[k] & m));
                }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = 16 * rt + i16;
            const bool ok = r < R && chan_ok;  // else read U's start, zeroed by the mask
            const uint16_t m = (uint16_t)keep_mask(ok);
            uint16_t v[4][W];
#pragma unroll
            for (int j = 0; j < 4; ++j) load_taps<W>(U + (ok ? ((int64_t)r * D + cbase + j) * W : 0), v[j]);
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = 2 * kp + (e >> 2);
                    ub[kp][rt][e] = __builtin_bit_cast(__bf16, (uint16_t)(k < W ? (v[e & 3][k] & m) : 0u));
                }
        }
        floatx4 du[W][RT];  // dU_k^T of the wave's 16 channels (rows) and 16-rank tiles
#pragma unroll
        for (int k = 0; k < W; ++k)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) du[k][rt] = floatx4{0.f, 0.f, 0.f, 0.f};

        for (int64_t s0 = 0; s0 < nsteps; s0 += P) {
            const int zs0 = (int)(s0 & 7);  // ring slot of step s0 (even)
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const int xcur = i % PX, xprv = (i + PX - 1) % PX;  // x slots of steps s, s-1
                const int gcur = i % PG, gnxt = (i + 1) % PG;       // dy slots of steps s, s+1
                const int ps = i & 1;
                const int64_t s = s0 + i;
                const int64_t nstep = nbeg + 16 * s;
                const int64_t n = nstep + tok;

                unsigned char *dxtp = dxt + ((s >> 1) & 1) * L::kDxt;  // this pair's dx tile
                float csn[4];  // ROPE: cos, sin of the next step's tokens (table load issued here)
                if constexpr (ROPE) rope_cs<4>(p, sp.pos_and_advance(starts, nstep + 16, tok), cbase, csn);
                if (ps == 0) {  // z rows two pairs ahead into the ring, the next pair fetched
                    write_zp(s / 2 + 2, zpf);
                    zpf = fetch_zp(s / 2 + 3);
                    if (s > 0) store_dx(s - 2);  // dx of the previous pair
                }

                // sequence masks: taps k <= back (dwc) and k < ahead (dx) stay in n's
                // sequence; bit j of win <-> token nstep - (W-1) + j.  A step with no
                // sequence start among its taps' tokens, inside the block's range, runs
                // a copy of the step without the masks (the test is wave-uniform).
                int back = W - 1, ahead = W;
                bool fast = nstep + 16 <= nend;
                {
                    const uint32_t win = __builtin_amdgcn_readfirstlane(starts.window(nstep - (W - 1)));
                    fast = fast && ((win >> 1) & ((1u << (2 * W + 13)) - 1u)) == 0u;
                    const uint32_t sb = (win >> (tok + 1)) & ((1u << (W - 1)) - 1u);  // starts in n-W+2 .. n
                    back = sb ? (W - 2) - (31 - __builtin_clz(sb)) : W - 1;
                    const uint32_t sa = (win >> (tok + W)) & ((1u << (W - 1)) - 1u);  // starts in n+1 .. n+W-1
                    ahead = sa ? 1 + __builtin_ctz(sa) : W;
                }
                // Each step forms dwc first (it is the last reader of x's previous
                // step), then issues the x refill, then forms the wave's part of dx (the
                // last reader of dy's current step) and issues the dy refill, so that
                // each load is in flight while the other half of the step runs.
                const unsigned char *zst = zring + 16 * (zs0 + i) * L::PZ;  // rows of step s
                auto dwc_part = [&](auto mask_tag) {
                    constexpr bool M = decltype(mask_tag)::value;
                    const uint32_t gc[2] = {gr[gcur].x, gr[gcur].y};
                    const uint32_t xc[2] = {xr[xcur].x, xr[xcur].y};
                    const uint32_t xp[2] = {xr[xprv].x, xr[xprv].y};
                    // dwc of every tap for the wave's channels: staged as dwc^T for dU,
                    // and by pairs of taps the B operand of dz^T += U dwc
                    const bool own = n < nend;  // tokens outside this block's range contribute nothing
                    floatx4 cz[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) cz[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp) {
                        uint32_t b4[4] = {0u, 0u, 0u, 0u};  // taps 2kp and 2kp+1 (zero past W)
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) {
                            const int k = 2 * kp + kk;
                            if (k >= W) continue;
                            uint32_t xk[2];
                            if (k == 0) {
                                xk[0] = xc[0];
                                xk[1] = xc[1];
                            } else {
                                shift_back2<W>(k, xc, xp, xk);
                            }
#pragma unroll
                            for (int i2 = 0; i2 < 2; ++i2) {
                                const uint32_t xv = (!M || (own && k <= back)) ? xk[i2] : 0u;
                                b4[2 * kk + i2] = pack_bf16x2(bf16_lo(gc[i2]) * bf16_lo(xv), bf16_hi(gc[i2]) * bf16_hi(xv));
                            }
                            *reinterpret_cast<uint2 *>(dwcT + k * 32 * L::PW + (16 * ps + tok) * L::PW + 8 * q) =
                                make_uint2(b4[2 * kk], b4[2 * kk + 1]);
                        }
                        const bf16x8 b = bf16x8_from_u32(b4);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            cz[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ub[kp][rt], b, cz[rt], 0, 0, 0);
                    }
                    // dz partials (rows r = 16rt + 4q + jj, column = token) for the block's sum
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        float4 *d = reinterpret_cast<float4 *>(dzb + (16 * ps + tok) * L::PD + 4 * (16 * rt + 4 * q));
                        *d = make_float4(cz[rt][0], cz[rt][1], cz[rt][2], cz[rt][3]);
                    }
                };
                auto dx_part = [&](auto mask_tag) {
                    constexpr bool M = decltype(mask_tag)::value;
                    const uint32_t gc[2] = {gr[gcur].x, gr[gcur].y};
                    const uint32_t gn[2] = {gr[gnxt].x, gr[gnxt].y};
                    // dx of the wave's 4 channels of every 8-channel chunk: the sum over
                    // every tap of w[n+k] dy[n+k] (rho entering as the accumulator of tap
                    // 0's product), into the pair's dx tile
                    float acc[4];
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const unsigned char *zrow_k = zst + (tok + k) * L::PZ;
                        bf16x8 zb[2];
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const uint2 *src = reinterpret_cast<const uint2 *>(zrow_k + 2 * (32 * c + 8 * q));
                            const uint2 a = src[0], b = src[1];
                            zb[c] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
                        }
                        uint32_t gk[2];
                        if (k == 0) {
                            gk[0] = gc[0];
                            gk[1] = gc[1];
                        } else {
                            shift_ahead2<W>(k, gc, gn, gk);
                            gk[0] = (!M || k < ahead) ? gk[0] : 0u;
                            gk[1] = (!M || k < ahead) ? gk[1] : 0u;
                        }
                        const float c0 = k == 0 ? p.rho : 0.f;
                        floatx4 cw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[k][0], zb[0],
                                                                             floatx4{c0, c0, c0, c0}, 0, 0, 0);
                        cw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[k][1], zb[1], cw, 0, 0, 0);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const float gv = (jj & 1) ? bf16_hi(gk[jj >> 1]) : bf16_lo(gk[jj >> 1]);
                            acc[jj] = k == 0 ? cw[jj] * gv : __builtin_fmaf(cw[jj], gv, acc[jj]);
                        }
                    }
                    *reinterpret_cast<uint2 *>(dxtp + (16 * ps + tok) * 256 + 16 * ((4 * slice + q) ^ tok) + 8 * HF) =
                        make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
                };
                if (fast) dwc_part(MaskTag<false>{}); else dwc_part(MaskTag<true>{});
                xr[xprv] = fetch_x(s + PX - 1);  // x of step s-1 is no longer read
                if constexpr (ROPE) turn_back(gr[gnxt], csn);  // the next step's dy, first read here
                if (fast) dx_part(MaskTag<false>{}); else dx_part(MaskTag<true>{});
                gr[gcur] = fetch_g(s + PG);      // dy of step s is no longer read

                if (ps == 1) {
                    lds_barrier();  // the pair's dx tile, dz partials and dwc^T rows of every wave
                    // dU_k^T[ch, r] += sum over the pair's 32 tokens of dwc_k^T[ch, tok] z[tok, r],
                    // operands re-read transposed (lane = channel / rank, registers = tokens)
                    const int trow = 8 * q + (i16 >> 2);
                    const int tcol = 4 * (i16 & 3);
                    const unsigned char *zpr = zring + 16 * (zs0 + i - 1) * L::PZ;  // the pair's 32 rows
                    bf16x8 zb[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        uint2 h[2];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) h[hh] = lds_read_tr(zpr + (trow + 4 * hh) * L::PZ + 2 * (16 * rt + tcol));
                        zb[rt] = __builtin_bit_cast(bf16x8, make_uint4(h[0].x, h[0].y, h[1].x, h[1].y));
                    }
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        uint2 h[2];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            h[hh] = lds_read_tr(dwcT + k * 32 * L::PW + (trow + 4 * hh) * L::PW + 2 * tcol);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(h[0].x, h[0].y, h[1].x, h[1].y));
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            du[k][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, zb[rt], du[k][rt], 0, 0, 0);
                    }
                    // dz of the pair: the 8 waves' partials summed, one fp32 atomic per
                    // (token, rank) below R and inside the block's range, each at an
                    // in-range offset of a resource based at the pair's first row
                    const int64_t npair0 = nbeg + 16 * (s - 1);
                    const __amdgpu_buffer_rsrc_t rdz =
                        make_stream(p.dzacc + group * p.dz_gstride + npair0 * R, (nend - npair0) * R * 4);
                    float v[4];
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int tl = wid + 8 * it;
                        const unsigned char *src = dz_all + tl * L::PD + 4 * lane;
                        float a = 0.f;
#pragma unroll
                        for (int w2 = 0; w2 < kTapWaves; ++w2) a += *reinterpret_cast<const float *>(src + w2 * L::kDzWave);
                        v[it] = a;
                    }
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int tl = wid + 8 * it;
                        // the token's row offset is wave-uniform: the scalar offset operand
                        if (lane < R && npair0 + tl < nend)
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                                v[it], rdz, 4 * lane, __builtin_amdgcn_readfirstlane(4 * tl * R), 0);
                    }
                    lds_barrier();  // every wave has read the exchange buffers before the next pair writes them
                }
            }
        }

        store_dx(nsteps - 2);  // dx of the last pair (finished before its second barrier)
        // dU tiles of the wave's taps -> the slice's staging tile in dU's memory
        // order [rank][channel*W + tap] (odd row pitch spreads the writes over the banks)
        __syncthreads();  // every wave is done with the loop's LDS regions
        float *dus = reinterpret_cast<float *>(lds + slice * L::kDuSlice);
#pragma unroll
        for (int k = 0; k < W; ++k)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int r = 16 * rt + i16;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) dus[r * L::kDuPitch + (8 * q + 4 * HF + jj) * W + k] = du[k][rt][jj];
            }
    };
    if (half == 0) walk(HalfTag<0>{}); else walk(HalfTag<1>{});
    __syncthreads();

    // the slice's tile added to dU with coalesced atomics (each wave
    // instruction covers 64 consecutive floats of one rank row); the two waves
    // of a slice take alternate groups of 4 ranks
    {
        const float *t0 = reinterpret_cast<const float *>(lds + slice * L::kDuSlice);
        const int nvalid = (int)((D - d0 < 32 ? D - d0 : 32) * W);  // floats of this slice inside D
        constexpr int kJ = (32 * W + kWave - 1) / kWave;
        float *dst = p.dU + tchunk * p.du_cstride + d0 * W;
#pragma unroll 1
        for (int rb = 4 * half; rb < R; rb += 8) {
            float v[4][kJ];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    const int idx = lane + kWave * j;
                    v[u][j] = idx < 32 * W ? t0[(rb + u) * L::kDuPitch + idx] : 0.f;
                }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    const int idx = lane + kWave * j;
                    if (rb + u < R && idx < nvalid) atomicAdd(dst + (int64_t)(rb + u) * DW + idx, v[u][j]);
                }
        }
    }
}

template <int W, bool ROPE>
const void *taps_kernel(bool zv) {
    return zv ? reinterpret_cast<const void *>(&lr_bwd_taps<W, true, ROPE>)
              : reinterpret_cast<const void *>(&lr_bwd_taps<W, false, ROPE>);
}

// Work split: ngroups blocks of 4 channel slices across D, token chunks of
// len tokens (whole pairs of steps) sized for `slots` resident blocks.
struct TapPlan {
    int64_t ngroups, len, tchunks;
};

TapPlan taps_plan(int64_t N, int64_t D, int64_t slots) {
    const int64_t ngroups = ((D + 31) / 32 + 3) / 4;
    const int64_t cap = walk_cap(D, 16 * kTapRing, 16 * (2 * kTapRing + 2));
    const int64_t len = walk_length(N, ngroups, slots, cap, 16 * kTapRing, 256);
    return TapPlan{ngroups, len, (N + len - 1) / len};
}

size_t det_dz_floats(const TapPlan &pl, int64_t N, int R) { return (((size_t)pl.ngroups * N * R + 3) / 4) * 4; }

template <int W, bool ROPE>
hipError_t taps_bwd(const LrProblem &pr, hipStream_t st, bool det) {
    LrParams p = make_params<BF16>(pr);
    const bool zv = p.R % 4 == 0;
    const int64_t nU = (int64_t)p.R * p.D * W;
    const int64_t nz = p.N * p.R;
    int64_t slots = kDetSlots;  // the reproducible split: one block per CU of a 256-CU device
    if (!det) {
        static const int bpc_v = blocks_per_cu(taps_kernel<W, ROPE>(true), kTapThreads);
        static const int bpc_g = blocks_per_cu(taps_kernel<W, ROPE>(false), kTapThreads);
        slots = (int64_t)device_cus() * (zv ? bpc_v : bpc_g);
    }
    const TapPlan pl = taps_plan(p.N, p.D, slots);
    float *du_sum = p.dU;
    int64_t nclear_dz = nz, nclear_du = nU;
    if (det) {  // regions of their own: dz per channel group, dU per token chunk
        p.dz_gstride = nz;
        p.du_cstride = nU;
        p.dU = p.dzacc + det_dz_floats(pl, p.N, p.R);
        nclear_dz = pl.ngroups * nz;
        nclear_du = pl.tchunks * nU;
    }
    hipError_t e = lowrank_zero2(p.dU, nclear_du, p.dzacc, nclear_dz, st);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(pl.tchunks * pl.ngroups));
    const int64_t nslices = (p.D + 31) / 32;
    if (zv)
        hipLaunchKernelGGL((lr_bwd_taps<W, true, ROPE>), grid, dim3(kTapThreads), 0, st, p, nslices, pl.len);
    else
        hipLaunchKernelGGL((lr_bwd_taps<W, false, ROPE>), grid, dim3(kTapThreads), 0, st, p, nslices, pl.len);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (det) {
        e = lowrank_sum_parts(p.dzacc, pl.ngroups, nz, nullptr, static_cast<uint16_t *>(p.dz), nz, st);
        if (e != hipSuccess) return e;
        return lowrank_sum_parts(p.dU, pl.tchunks, nU, du_sum, nullptr, nU, st);
    }
    return lowrank_round_bf16(p.dzacc, static_cast<uint16_t *>(p.dz), nz, st);
}

}  // namespace

bool lowrank_bwd_taps_supported(Dtype dt, int64_t D, int32_t W, int32_t R) {
    if (dt != Dtype::BF16 || W < 2 || W > 4 || R <= 32 || R > 64) return false;
    return walk_cap(D, 16 * kTapRing, 16 * (2 * kTapRing + 2)) >= 16 * kTapRing;
}

hipError_t lowrank_bwd_taps(const LrProblem &pr, hipStream_t st, bool det) {
    switch (pr.W) {
        case 2: return taps_bwd<2, false>(pr, st, det);
        case 3: return taps_bwd<3, false>(pr, st, det);
        case 4: return taps_bwd<4, false>(pr, st, det);
        default: return hipErrorInvalidValue;
    }
}

hipError_t lowrank_bwd_taps_rope(const LrProblem &pr, hipStream_t st) {
    switch (pr.W) {
        case 2: return taps_bwd<2, true>(pr, st, false);
        case 3: return taps_bwd<3, true>(pr, st, false);
        case 4: return taps_bwd<4, true>(pr, st, false);
        default: return hipErrorInvalidValue;
    }
}

size_t lowrank_bwd_taps_det_workspace(int64_t N, int64_t D, int32_t W, int32_t R) {
    const TapPlan pl = taps_plan(N, D, kDetSlots);
    const size_t bytes = (det_dz_floats(pl, N, R) + (size_t)pl.tchunks * R * D * W) * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

}  // namespace dsc
