// stream.hip -- a plain streaming kernel for gfx950: the practical HBM
// ceiling against which the convolution kernels are read.  It is a
// measurement aid, not part of the operation: it reads one buffer and writes
// another in 16-byte units per lane, with the load and store cache policies,
// the number of loads in flight and the order of the units as choices, so
// that the fastest recipe for a given read / write mix can be found on the
// device itself.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "dsc_kernels.h"

namespace dsc {
namespace {

constexpr int kStreamBlock = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4 *p) {
    if constexpr (NT) {
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st16(uint4 *p, uint4 v) {
    if constexpr (NT) {
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
    } else {
        *p = v;
    }
}

// Unit i (16 bytes) is read when i < nr and written when i < nw (the value
// written is the one read, or the unit index where nothing is read).  Every
// thread takes U units per round.  Interleaved order (CHUNKED false): unit
// tid + j*S of round j, S = the grid's threads, so each wave instruction
// covers 1 KB and the grid sweeps the buffers front to back.  Chunked order:
// block b takes the contiguous range [b*per, (b+1)*per) in 4*U KB rounds.
// A read-only stream keeps its loads alive through an xor that is stored (to
// sink) only when it equals a value no input of the probe produces.
template <int U, bool LNT, bool SNT, bool CHUNKED>
__global__ __launch_bounds__(kStreamBlock) void stream_kernel(const uint4 *__restrict__ src, int64_t nr,
                                                              uint4 *__restrict__ dst, int64_t nw, int64_t per,
                                                              uint4 *sink) {
    const int64_t n = nr > nw ? nr : nw;
    int64_t base, step, end;
    if constexpr (CHUNKED) {
        base = (int64_t)blockIdx.x * per + threadIdx.x;
        step = kStreamBlock;
        end = min((int64_t)(blockIdx.x + 1) * per, n);
    } else {
        base = (int64_t)blockIdx.x * kStreamBlock + threadIdx.x;
        step = (int64_t)gridDim.x * kStreamBlock;
        end = n;
    }
    uint32_t acc = 0u;
    int64_t i = base;
    for (; i + (U - 1) * step < end; i += U * step) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + u * step;
            v[u] = j < nr ? ld16<LNT>(src + j) : make_uint4((uint32_t)j, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + u * step;
            if (j < nw) st16<SNT>(dst + j, v[u]);
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    for (; i < end; i += step) {
        const uint4 v = i < nr ? ld16<LNT>(src + i) : make_uint4((uint32_t)i, 0u, 0u, 0u);
        if (i < nw) st16<SNT>(dst + i, v);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (nw == 0 && acc == 0x9e3779b9u && sink) *sink = make_uint4(acc, 0u, 0u, 0u);
}

template <int U, bool LNT, bool SNT>
hipError_t launch_order(bool chunked, const uint4 *src, int64_t nr, uint4 *dst, int64_t nw, int64_t blocks,
                        uint4 *sink, hipStream_t st) {
    const int64_t n = nr > nw ? nr : nw;
    const int64_t per = ((n + blocks - 1) / blocks + kStreamBlock - 1) / kStreamBlock * kStreamBlock;
    if (chunked)
        hipLaunchKernelGGL((stream_kernel<U, LNT, SNT, true>), dim3((unsigned)blocks), dim3(kStreamBlock), 0, st, src,
                           nr, dst, nw, per, sink);
    else
        hipLaunchKernelGGL((stream_kernel<U, LNT, SNT, false>), dim3((unsigned)blocks), dim3(kStreamBlock), 0, st,
                           src, nr, dst, nw, per, sink);
    return hipGetLastError();
}

template <int U>
hipError_t launch_policy(bool lnt, bool snt, bool chunked, const uint4 *src, int64_t nr, uint4 *dst, int64_t nw,
                         int64_t blocks, uint4 *sink, hipStream_t st) {
    if (lnt) {
        return snt ? launch_order<U, true, true>(chunked, src, nr, dst, nw, blocks, sink, st)
                   : launch_order<U, true, false>(chunked, src, nr, dst, nw, blocks, sink, st);
    }
    return snt ? launch_order<U, false, true>(chunked, src, nr, dst, nw, blocks, sink, st)
               : launch_order<U, false, false>(chunked, src, nr, dst, nw, blocks, sink, st);
}

}  // namespace

int64_t stream_default_blocks() {
    static const int bpc = blocks_per_cu(reinterpret_cast<const void *>(&stream_kernel<4, false, false, false>),
                                         kStreamBlock);
    return (int64_t)device_cus() * bpc;
}

hipError_t stream_probe(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes, int unroll, bool lnt,
                        bool snt, bool chunked, int64_t blocks, hipStream_t st) {
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    if (nr == 0 && nw == 0) return hipSuccess;
    if (blocks <= 0) blocks = stream_default_blocks();
    const uint4 *s = static_cast<const uint4 *>(src);
    uint4 *d = static_cast<uint4 *>(dst);
    uint4 *sink = d;
    switch (unroll) {
        case 1: return launch_policy<1>(lnt, snt, chunked, s, nr, d, nw, blocks, sink, st);
        case 2: return launch_policy<2>(lnt, snt, chunked, s, nr, d, nw, blocks, sink, st);
        case 4: return launch_policy<4>(lnt, snt, chunked, s, nr, d, nw, blocks, sink, st);
        case 8: return launch_policy<8>(lnt, snt, chunked, s, nr, d, nw, blocks, sink, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsc
