// dsc_common.h -- device helpers shared by the dynamic short convolution
// kernels (gfx950, wave64).  Internal to libdsc.so.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

namespace dsc {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------- element types

// Storage tags.  Values are always widened to fp32 for arithmetic.
struct F32 {
    using store_t = float;
    static constexpr int kVec = 4;  // elements per 16-byte vector
};
struct BF16 {
    using store_t = uint16_t;
    static constexpr int kVec = 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
    return (uint16_t)(pack_bf16x2(a, 0.f) & 0xffffu);
}

// Global loads and stores of 4, 8 and 16 bytes, optionally with the
// nontemporal (streaming) cache policy: data that is read or written once per
// launch, where the policy measured 15-20% faster HBM streaming on MI355X.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ uint4 ld_u4(const void *p) {
    if constexpr (NT) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4 *>(p)));
    else return *static_cast<const uint4 *>(p);
}
template <bool NT>
__device__ __forceinline__ uint2 ld_u2(const void *p) {
    if constexpr (NT) return __builtin_bit_cast(uint2, __builtin_nontemporal_load(static_cast<const u32x2 *>(p)));
    else return *static_cast<const uint2 *>(p);
}
template <bool NT>
__device__ __forceinline__ uint32_t ld_u1(const void *p) {
    if constexpr (NT) return __builtin_nontemporal_load(static_cast<const uint32_t *>(p));
    else return *static_cast<const uint32_t *>(p);
}
template <bool NT>
__device__ __forceinline__ void st_u4(void *p, uint4 v) {
    if constexpr (NT) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), static_cast<u32x4 *>(p));
    else *static_cast<uint4 *>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void st_u2(void *p, uint2 v) {
    if constexpr (NT) __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), static_cast<u32x2 *>(p));
    else *static_cast<uint2 *>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void st_u1(void *p, uint32_t v) {
    if constexpr (NT) __builtin_nontemporal_store(v, static_cast<uint32_t *>(p));
    else *static_cast<uint32_t *>(p) = v;
}

// 16-byte vector of VEC elements <-> VEC floats.
template <class E>
struct Vec16;

template <>
struct Vec16<F32> {
    __device__ __forceinline__ static void load(const void *p, float (&v)[4]) {
        float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    template <bool NT = false>
    __device__ __forceinline__ static void store(void *p, const float (&v)[4]) {
        st_u4<NT>(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                __float_as_uint(v[3])));
    }
};

template <>
struct Vec16<BF16> {
    __device__ __forceinline__ static void load(const void *p, float (&v)[8]) {
        uint4 q = *reinterpret_cast<const uint4 *>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
        v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    template <bool NT = false>
    __device__ __forceinline__ static void store(void *p, const float (&v)[8]) {
        uint4 q;
        q.x = pack_bf16x2(v[0], v[1]);
        q.y = pack_bf16x2(v[2], v[3]);
        q.z = pack_bf16x2(v[4], v[5]);
        q.w = pack_bf16x2(v[6], v[7]);
        st_u4<NT>(p, q);
    }
};

// One element widened to fp32.
template <class E>
__device__ __forceinline__ float load_elem(const typename E::store_t *p) {
    if constexpr (sizeof(typename E::store_t) == 4) return *p;
    else return __uint_as_float((uint32_t)*p << 16);
}

// Largest power of two <= 16 dividing n.
__host__ __device__ constexpr int pow2_align(int n) {
    return (n % 16 == 0) ? 16 : (n % 8 == 0) ? 8 : (n % 4 == 0) ? 4 : (n % 2 == 0) ? 2 : 1;
}

// Contiguous span of NE elements starting at an address aligned to ALIGN bytes:
// loaded / stored with the widest aligned accesses.
// NE elements kept as raw 32-bit words (bf16 pairs or fp32), widened on use.
template <class E, int NE>
struct RawSpan {
    using S = typename E::store_t;
    static constexpr int kBytes = NE * (int)sizeof(S);
    static constexpr int kWords = (kBytes + 3) / 4;
    template <int ALIGN, bool NT = false>
    __device__ __forceinline__ static void load(const S *p, uint32_t (&w)[kWords]) {
        constexpr int A = ALIGN < kBytes ? ALIGN : pow2_align(kBytes);
        if constexpr (A < 4) {  // 2-byte elements, 2-byte aligned
            const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
            for (int i = 0; i < kWords; ++i) {
                const uint32_t lo = h[2 * i];
                const uint32_t hi = 2 * i + 1 < NE ? (uint32_t)h[2 * i + 1] : 0u;
                w[i] = lo | (hi << 16);
            }
            return;
        }
        constexpr int WPL = A >= 16 ? 4 : (A >= 4 ? A / 4 : 1);  // words per load
#pragma unroll
        for (int i = 0; i < kWords; i += WPL) {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(p) + i;
            if constexpr (WPL == 4) {
                const uint4 v = ld_u4<NT>(q);
                w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
            } else if constexpr (WPL == 2) {
                const uint2 v = ld_u2<NT>(q);
                w[i] = v.x; w[i + 1] = v.y;
            } else {
                w[i] = ld_u1<NT>(q);
            }
        }
    }
    __device__ __forceinline__ static float at(const uint32_t (&w)[kWords], int i) {
        if constexpr (sizeof(S) == 4) return __uint_as_float(w[i]);
        else return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    }
};

template <class E, int NE>
struct Span {
    using S = typename E::store_t;
    static constexpr int kBytes = NE * (int)sizeof(S);

    template <int ALIGN>
    __device__ __forceinline__ static void load(const S *p, float (&v)[NE]) {
        constexpr int A = ALIGN < kBytes ? ALIGN : pow2_align(kBytes);
        constexpr int PER = A / (int)sizeof(S) > 0 ? A / (int)sizeof(S) : 1;
        static_assert(NE % PER == 0, "span split");
#pragma unroll
        for (int i = 0; i < NE; i += PER) {
            if constexpr (A >= 16) {
                uint4 q = *reinterpret_cast<const uint4 *>(p + i);
                unpack<4>(&q.x, v, i);
            } else if constexpr (A == 8) {
                uint2 q = *reinterpret_cast<const uint2 *>(p + i);
                unpack<2>(&q.x, v, i);
            } else if constexpr (A == 4) {
                uint32_t q = *reinterpret_cast<const uint32_t *>(p + i);
                unpack<1>(&q, v, i);
            } else {
                v[i] = widen(p[i]);
            }
        }
    }

    template <int ALIGN, bool NT = false>
    __device__ __forceinline__ static void store(S *p, const float (&v)[NE]) {
        constexpr int A = ALIGN < kBytes ? ALIGN : pow2_align(kBytes);
        constexpr int PER = A / (int)sizeof(S) > 0 ? A / (int)sizeof(S) : 1;
#pragma unroll
        for (int i = 0; i < NE; i += PER) {
            if constexpr (A >= 16) {
                uint4 q;
                pack<4>(&q.x, v, i);
                st_u4<NT>(p + i, q);
            } else if constexpr (A == 8) {
                uint2 q;
                pack<2>(&q.x, v, i);
                st_u2<NT>(p + i, q);
            } else if constexpr (A == 4) {
                uint32_t q;
                pack<1>(&q, v, i);
                st_u1<NT>(p + i, q);
            } else {
                p[i] = narrow(v[i]);
            }
        }
    }

   private:
    __device__ __forceinline__ static float widen(S s) {
        if constexpr (sizeof(S) == 4) return __builtin_bit_cast(float, s);
        else return __uint_as_float((uint32_t)s << 16);
    }
    __device__ __forceinline__ static S narrow(float f) {
        if constexpr (sizeof(S) == 4) return f;
        else return to_bf16(f);
    }
    template <int NW>
    __device__ __forceinline__ static void unpack(const uint32_t *q, float (&v)[NE], int i) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if constexpr (sizeof(S) == 4) {
                v[i + j] = __uint_as_float(q[j]);
            } else {
                v[i + 2 * j] = bf16_lo(q[j]);
                v[i + 2 * j + 1] = bf16_hi(q[j]);
            }
        }
    }
    template <int NW>
    __device__ __forceinline__ static void pack(uint32_t *q, const float (&v)[NE], int i) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            if constexpr (sizeof(S) == 4) q[j] = __float_as_uint(v[i + j]);
            else q[j] = pack_bf16x2(v[i + 2 * j], v[i + 2 * j + 1]);
        }
    }
};

// Orders a wave's LDS writes before its later LDS reads at compile time.
// Lanes that read what other lanes of the same wave wrote need it: without
// it the compiler may move a read above a write whose address differs in
// every single lane.  It emits no instruction (LDS operations of one wave
// execute in issue order).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

// All ones when ok, else zero, hidden from the optimizer: a load whose
// value is masked by it stays unconditional (a select on the loaded value
// would be turned into a branch around the load, and a loop of such loads
// then waits for each one in turn).
__device__ __forceinline__ uint32_t keep_mask(bool ok) {
    uint32_t m = ok ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(m));
    return m;
}

// Workgroup barrier for waves that exchange data through LDS only: the
// wave's LDS operations complete before it (lgkmcnt 0) and no LDS access
// moves across it.  __syncthreads also waits for every global load and store
// the wave has in flight (vmcnt 0), which drains a prefetch ring and waits
// for store acknowledgements at every barrier; this one leaves them in
// flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ----------------------------------------------------------- buffer access

// Raw buffer resources: loads outside a resource's range read zero and
// stores outside it are dropped by the hardware, which replaces per-lane
// bounds branches on the streaming paths.
constexpr uint32_t kBufferWord3 = 0x00020000u;  // gfx9-family raw buffer format

// Streams with one resource per walk: a lane's offset is its place inside a
// step plus the step's offset, both below 2^30 (the launchers cap the walk
// length so that this holds).  Lanes with nothing to move start at kFar; the
// resource size is clamped to kFar, so they stay out of range at every step
// and no offset comes near the top of the 32-bit range.  Atomics never rely
// on the range check: they are issued only by lanes whose offset is in range.
constexpr uint32_t kFar = 0xc0000000u;
constexpr int64_t kStreamSpan = 0x3fffffff;  // largest in-walk offset

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_stream(const void *base, int64_t bytes) {
    const int64_t b = bytes < 0 ? 0 : (bytes > (int64_t)kFar ? (int64_t)kFar : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)b, kBufferWord3);
}

// NT: the nontemporal (streaming) cache policy, for streams read or written
// once per launch in whole cache lines.
template <bool NT = false>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}

template <bool NT = false>
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? 2 : 0));
}

template <bool NT = false>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                           r, off, 0, NT ? 2 : 0);
}

// ----------------------------------------------------------- sequences

// Sequence [start, end) on the flattened token axis that contains token n.
// Without offsets every row of T tokens is one sequence; otherwise binary
// search of cu[0..n_seqs] (cu[0] = 0, cu[n_seqs] = N, increasing).
struct SeqMap {
    const int32_t *cu;
    int32_t n_seqs;
    int64_t T;

    __device__ __forceinline__ void find(int64_t n, int64_t &start, int64_t &end) const {
        if (cu == nullptr) {
            start = (n / T) * T;
            end = start + T;
            return;
        }
        int lo = 0, hi = n_seqs;  // invariant: cu[lo] <= n < cu[hi]
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if ((int64_t)cu[mid] <= n) lo = mid;
            else hi = mid;
        }
        start = cu[lo];
        end = cu[lo + 1];
    }
};

// Per-wave bit map of sequence starts over the tokens [base, base + 32*kWords),
// kept in LDS and built once before a wave's token walk, so the walk itself
// issues no memory loads besides its data stream (which keeps the compiler's
// load counters exact and the prefetch in flight).  Bit i is set when token
// base + i is the first token of a sequence, or is N (one past the end).
template <int kWords>
struct StartBits {
    uint32_t *words;  // LDS, owned by one wave
    int64_t base;

    // All 64 lanes of the wave call this; it ends with a wave LDS fence, so
    // the wave can read the map right after.
    __device__ void build(uint32_t *lds_words, const SeqMap &m, int64_t N, int64_t first_token, int lane) {
        words = lds_words;
        base = first_token;
        const int64_t hi = base + 32 * (int64_t)kWords;
        // The wave's LDS operations execute in issue order; the fences keep
        // the compiler from reordering the zeroing, the marking by other
        // lanes and the caller's reads.
        for (int i = lane; i < kWords; i += kWave) words[i] = 0u;
        wave_lds_fence();
        auto mark = [&](int64_t t) {
            if (t >= base && t < hi) {
                const int64_t o = t - base;
                atomicOr(&words[o >> 5], 1u << (o & 31));
            }
        };
        if (m.cu == nullptr) {
            const int64_t lo = base > 0 ? base : 0;
            const int64_t first = ((lo + m.T - 1) / m.T) * m.T;
            for (int64_t t = first + (int64_t)lane * m.T; t < hi && t <= N; t += (int64_t)kWave * m.T) mark(t);
        } else {
            int lo = 0, hi_i = m.n_seqs;  // first index with cu[i] >= base
            if ((int64_t)m.cu[0] >= base) {
                hi_i = 0;
            } else {
                while (hi_i - lo > 1) {
                    const int mid = (lo + hi_i) >> 1;
                    if ((int64_t)m.cu[mid] >= base) hi_i = mid;
                    else lo = mid;
                }
            }
            for (int j = hi_i + lane; j <= m.n_seqs; j += kWave) {
                const int64_t t = m.cu[j];
                if (t >= hi) break;
                mark(t);
            }
        }
        wave_lds_fence();  // the caller's window reads see every lane's marks
    }

    // 32 bits of the map starting at token t (base <= t, t + 32 <= base + 32*kWords).
    __device__ __forceinline__ uint32_t window(int64_t t) const {
        const int64_t o = t - base;
        const int w = (int)(o >> 5), b = (int)(o & 31);
        const uint32_t lo = words[w];
        const uint32_t hi = b ? words[w + 1] : 0u;
        return b ? (lo >> b) | (hi << (32 - b)) : lo;
    }
};

// Workgroup id remapped so that consecutive logical blocks run on the same
// XCD: the dispatcher hands block b to XCD b % 8, and neighbouring tiles share
// halo rows that then stay in that XCD's L2.  Bijective for any grid size.
__device__ __forceinline__ int64_t xcd_block_id(int64_t b, int64_t nblocks) {
    constexpr int kXcd = 8;
    int64_t q = nblocks / kXcd, r = nblocks % kXcd;
    int64_t x = b % kXcd;
    int64_t start = x * q + (x < r ? x : r);
    return start + b / kXcd;
}

// ------------------------------------------------------- rotary embedding
// Pair j of a chunk is (v[2j], v[2j+1]); a table row holds cos, sin of each
// pair of a head in turn ("RoFormer: Enhanced Transformer with Rotary Position
// Embedding", Su et al., Section 3.4.2).

// cos, sin of a thread's VEC/2 pairs at one position (VEC floats, 16-byte
// aligned because a chunk starts at a multiple of VEC inside its head).
template <int VEC>
__device__ __forceinline__ void load_turn(const float *t, float (&cs)[VEC]) {
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(t + i);
        cs[i] = v.x; cs[i + 1] = v.y; cs[i + 2] = v.z; cs[i + 3] = v.w;
    }
}

// cs <- an (x) cs pair by pair: cos and sin of the sum of the two angles.
template <int VEC>
__device__ __forceinline__ void compose(float (&cs)[VEC], const float (&an)[VEC]) {
#pragma unroll
    for (int j = 0; j < VEC / 2; ++j) {
        const float c1 = an[2 * j], s1 = an[2 * j + 1], c2 = cs[2 * j], s2 = cs[2 * j + 1];
        cs[2 * j] = c1 * c2 - s1 * s2;
        cs[2 * j + 1] = s1 * c2 + c1 * s2;
    }
}

template <int VEC>
__device__ __forceinline__ void set_identity(float (&cs)[VEC]) {
#pragma unroll
    for (int j = 0; j < VEC / 2; ++j) {
        cs[2 * j] = 1.f;
        cs[2 * j + 1] = 0.f;
    }
}

// Turns every pair (v[2j], v[2j+1]) by the angle whose cos, sin are
// cs[2j], cs[2j+1]; INV turns by the opposite angle (the transpose).
template <int VEC, bool INV>
__device__ __forceinline__ void turn(float (&v)[VEC], const float (&cs)[VEC]) {
#pragma unroll
    for (int j = 0; j < VEC / 2; ++j) {
        const float c = cs[2 * j], s = INV ? -cs[2 * j + 1] : cs[2 * j + 1];
        const float a = v[2 * j], b = v[2 * j + 1];
        v[2 * j] = a * c - b * s;
        v[2 * j + 1] = b * c + a * s;
    }
}

// ----------------------------------------------------------- launch sizing (host)

// Compute units of the current device (all devices of a process are taken
// to be alike).
inline int device_cus() {
    static std::atomic<int> cus{0};
    int n = cus.load(std::memory_order_relaxed);
    if (n == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus.store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of `kernel` (`threads` per block, static LDS only) resident per
// compute unit, from the runtime's occupancy calculator.
inline int blocks_per_cu(const void *kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

}  // namespace dsc
