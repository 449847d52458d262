/*
 * dsc_bench.h -- measurement aid of libdsc.so: a plain streaming kernel that
 * gives the practical HBM ceiling of the device, against which the
 * convolution kernels of dsc.h are read.  It computes nothing of the
 * operation.
 */
#ifndef DSC_BENCH_H
#define DSC_BENCH_H

#include "dsc.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads read_bytes from src and writes write_bytes to dst in 16-byte units
 * (unit i is read when i < read_bytes/16 and written when i < write_bytes/16;
 * the value written is the unit read, or its index when nothing is read), so
 * one launch moves a chosen mix of read and written bytes.
 *
 *   stream       hipStream_t as void* (NULL: the null stream), asynchronous.
 *   src, dst     DEVICE pointers, 16-byte aligned, not overlapping.  dst is
 *                required even when write_bytes = 0 (a read-only stream
 *                keeps its loads alive through a store to dst[0] that a
 *                value no input produces would trigger).  src may be NULL
 *                when read_bytes = 0.
 *   read_bytes, write_bytes   multiples of 16, each below 2^40.
 *   unroll       16-byte loads a thread keeps in flight: 1, 2, 4 or 8.
 *   load_nt, store_nt   1: nontemporal (streaming) cache policy, 0: default.
 *   chunked      0: unit tid + j*S of round j (S = the grid's threads);
 *                1: each workgroup takes one contiguous range of units.
 *   blocks       workgroups of 256 threads; 0 = one round of resident
 *                workgroups on the current device (compute units x
 *                workgroups per unit).
 * Returns DSC_ERR_SHAPE / DSC_ERR_NULL / DSC_ERR_ALIGNMENT / DSC_ERR_ALIAS
 * before any HIP call on bad arguments, DSC_ERR_HIP if the launch fails.
 */
DSC_API dsc_status dsc_bench_stream(void *stream, const void *src, int64_t read_bytes, void *dst,
                                    int64_t write_bytes, int32_t unroll, int32_t load_nt, int32_t store_nt,
                                    int32_t chunked, int64_t blocks);

#ifdef __cplusplus
}
#endif

#endif /* DSC_BENCH_H */
