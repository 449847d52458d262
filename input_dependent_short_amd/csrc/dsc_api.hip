// dsc_api.hip -- the C ABI of libdsc.so (declared in include/dsc.h):
// argument validation, then one launch sequence on the caller's stream.
// Every precondition that the host can check is checked before the first HIP
// call, so invalid calls never touch the device.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/dsc.h"
#include "../../include/dsc_bench.h"
#include "dsc_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

dsc_status fail(dsc_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

dsc_status ok() {
    g_last_error[0] = '\0';
    return DSC_SUCCESS;
}

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// No output range may intersect an input range or another output range.
dsc_status check_alias(const Range *in, int nin, const Range *out, int nout) {
    for (int i = 0; i < nout; ++i) {
        if (out[i].hi <= out[i].lo) continue;
        for (int j = 0; j < nin; ++j)
            if (in[j].hi > in[j].lo && out[i].lo < in[j].hi && in[j].lo < out[i].hi)
                return fail(DSC_ERR_ALIAS, "output %s overlaps input %s", out[i].name, in[j].name);
        for (int j = i + 1; j < nout; ++j)
            if (out[j].hi > out[j].lo && out[i].lo < out[j].hi && out[j].lo < out[i].hi)
                return fail(DSC_ERR_ALIAS, "outputs %s and %s overlap", out[i].name, out[j].name);
    }
    return DSC_SUCCESS;
}

Range rng(const char *name, const void *p, size_t bytes) {
    return Range{name, (uintptr_t)p, (uintptr_t)p + bytes};
}

size_t esize(int dtype) { return dtype == DSC_BF16 ? 2 : 4; }

dsc_status check_common(int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                        const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual) {
    if (dtype != DSC_FP32 && dtype != DSC_BF16) return fail(DSC_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (B < 0 || T < 0 || D < 1) return fail(DSC_ERR_SHAPE, "B, T must be >= 0 and D >= 1 (got %lld, %lld, %lld)",
                                             (long long)B, (long long)T, (long long)D);
    if (T > 0 && B > (int64_t)INT32_MAX / T)  // B*T > 2^31-1, tested without forming the product
        return fail(DSC_ERR_SHAPE, "B*T tokens exceed 2^31-1 (B = %lld, T = %lld)", (long long)B, (long long)T);
    if (D > ((int64_t)1 << 24)) return fail(DSC_ERR_SHAPE, "D = %lld too large", (long long)D);
    if (W < 1 || W > 8) return fail(DSC_ERR_SHAPE, "W must be in 1..8 (got %d)", W);
    const int vec = dtype == DSC_BF16 ? 8 : 4;
    if (D % vec) return fail(DSC_ERR_SHAPE, "D = %lld must be a multiple of %d for this dtype", (long long)D, vec);
    if (residual != 0 && residual != 1) return fail(DSC_ERR_SHAPE, "residual must be 0 or 1");
    if (B * T == 0) return DSC_SUCCESS;  // empty batch: cu_seqlens is not read
    if ((cu_seqlens == nullptr) != (n_seqs == 0))
        return fail(DSC_ERR_SHAPE, "cu_seqlens and n_seqs disagree (NULL pointer iff n_seqs == 0)");
    if (n_seqs < 0 || n_seqs > B * T) return fail(DSC_ERR_SHAPE, "n_seqs = %d out of range", n_seqs);
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u)) return fail(DSC_ERR_ALIGNMENT, "cu_seqlens not 4-byte aligned");
    return DSC_SUCCESS;
}

#define DSC_TRY(expr)                        \
    do {                                     \
        dsc_status st_ = (expr);             \
        if (st_ != DSC_SUCCESS) return st_;  \
    } while (0)

dsc_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(DSC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

dsc_status dsc_headwise_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                            int32_t H, const void *x, const void *w, const int32_t *cu_seqlens,
                            int32_t n_seqs, int32_t residual, void *y) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (H < 1 || D % H) return fail(DSC_ERR_SHAPE, "H = %d must divide D = %lld", H, (long long)D);
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    if (B * T == 0) return ok();  // empty batch: nothing to compute
    if (!x || !w || !y) return fail(DSC_ERR_NULL, "x, w and y are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("w", w, N * (D / H) * W * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("y", y, N * D * es)};
    DSC_TRY(check_alias(in, 3, out, 1));
    dsc::HwProblem p{dt, B * T, T, D, W, H, x, w, nullptr, y, nullptr, nullptr, cu_seqlens, n_seqs, residual};
    return launched(dsc::headwise_fwd(p, (hipStream_t)stream), "dsc_headwise_fwd launch");
}

dsc_status dsc_headwise_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                            int32_t H, const void *x, const void *w, const void *dy,
                            const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                            void *dx, void *dw) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (H < 1 || D % H) return fail(DSC_ERR_SHAPE, "H = %d must divide D = %lld", H, (long long)D);
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    if (B * T == 0) return ok();  // empty batch: dx and dw have no elements
    if (!x || !w || !dy || !dx || !dw) return fail(DSC_ERR_NULL, "x, w, dy, dx and dw are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(dy) || !aligned16(dx) || !aligned16(dw))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const size_t wb = N * (D / H) * W * es;
    const Range in[] = {rng("x", x, N * D * es), rng("w", w, wb), rng("dy", dy, N * D * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("dx", dx, N * D * es), rng("dw", dw, wb)};
    DSC_TRY(check_alias(in, 4, out, 2));
    dsc::HwProblem p{dt, B * T, T, D, W, H, x, w, dy, nullptr, dx, dw, cu_seqlens, n_seqs, residual};
    return launched(dsc::headwise_bwd(p, (hipStream_t)stream), "dsc_headwise_bwd launch");
}

dsc_status dsc_rope_table(void *stream, int64_t max_pos, int32_t head_dim, double base, float *table) {
    if (max_pos < 0 || max_pos > INT32_MAX) return fail(DSC_ERR_SHAPE, "max_pos = %lld out of range", (long long)max_pos);
    if (head_dim < 2 || head_dim % 2 || head_dim > (1 << 16))
        return fail(DSC_ERR_SHAPE, "head_dim = %d must be even, in 2..65536", head_dim);
    if (!(base > 0.0) || base > 1e300) return fail(DSC_ERR_SHAPE, "base must be positive and finite");
    if (max_pos * (head_dim / 2) > (int64_t)INT32_MAX * 64) return fail(DSC_ERR_SHAPE, "table too large");
    if (max_pos == 0) return ok();
    if (!table) return fail(DSC_ERR_NULL, "table is required");
    if (!aligned16(table)) return fail(DSC_ERR_ALIGNMENT, "table must be 16-byte aligned");
    return launched(dsc::rope_table(max_pos, head_dim, base, table, (hipStream_t)stream), "dsc_rope_table launch");
}

namespace {

// Rotation arguments of the fused head-wise + rotary calls.  A table row must
// exist for every position a token can have: T without cu_seqlens, else the
// whole packed batch B*T (a sequence can be that long).
dsc_status check_rope(int dtype, int64_t B, int64_t T, int64_t D, const int32_t *cu_seqlens, int64_t rot,
                      int32_t head_dim, const float *table, int64_t max_pos) {
    if (head_dim < 2 || head_dim % 2 || head_dim > (1 << 16))
        return fail(DSC_ERR_SHAPE, "head_dim = %d must be even, in 2..65536", head_dim);
    const int vec = dtype == DSC_BF16 ? 8 : 4;
    if (head_dim % vec)
        return fail(DSC_ERR_UNSUPPORTED, "head_dim = %d must be a multiple of %d for this dtype", head_dim, vec);
    if (rot < 0 || rot > D || rot % head_dim)
        return fail(DSC_ERR_SHAPE, "rot = %lld must be a multiple of head_dim in 0..D", (long long)rot);
    if (rot == 0 || B * T == 0) return DSC_SUCCESS;
    const int64_t need = cu_seqlens ? B * T : T;
    if (max_pos < need)
        return fail(DSC_ERR_SHAPE, "max_pos = %lld: the table needs a row for each of %lld positions",
                    (long long)max_pos, (long long)need);
    if (max_pos > INT32_MAX / head_dim) return fail(DSC_ERR_SHAPE, "max_pos * head_dim exceeds 2^31-1");
    if (!table) return fail(DSC_ERR_NULL, "table is required when rot > 0");
    if (!aligned16(table)) return fail(DSC_ERR_ALIGNMENT, "table must be 16-byte aligned");
    return DSC_SUCCESS;
}

}  // namespace

dsc_status dsc_headwise_rope_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                 int32_t H, const void *x, const void *w, const int32_t *cu_seqlens,
                                 int32_t n_seqs, int32_t residual, int64_t rot, int32_t head_dim,
                                 const float *table, int64_t max_pos, void *y) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (H < 1 || D % H) return fail(DSC_ERR_SHAPE, "H = %d must divide D = %lld", H, (long long)D);
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    DSC_TRY(check_rope(dtype, B, T, D, cu_seqlens, rot, head_dim, table, max_pos));
    if (B * T == 0) return ok();
    if (!x || !w || !y) return fail(DSC_ERR_NULL, "x, w and y are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("w", w, N * (D / H) * W * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0),
                        rng("table", table, rot ? (size_t)max_pos * head_dim * 4u : 0)};
    const Range out[] = {rng("y", y, N * D * es)};
    DSC_TRY(check_alias(in, 4, out, 1));
    dsc::HwProblem p{dt, B * T, T, D, W, H, x, w, nullptr, y, nullptr, nullptr, cu_seqlens, n_seqs, residual,
                     rot, head_dim, table, max_pos};
    if (rot == 0) return launched(dsc::headwise_fwd(p, (hipStream_t)stream), "dsc_headwise_rope_fwd launch");
    return launched(dsc::headwise_rope_fwd(p, (hipStream_t)stream), "dsc_headwise_rope_fwd launch");
}

dsc_status dsc_headwise_rope_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                 int32_t H, const void *x, const void *w, const void *dy,
                                 const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, int64_t rot,
                                 int32_t head_dim, const float *table, int64_t max_pos, void *dx, void *dw) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (H < 1 || D % H) return fail(DSC_ERR_SHAPE, "H = %d must divide D = %lld", H, (long long)D);
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    DSC_TRY(check_rope(dtype, B, T, D, cu_seqlens, rot, head_dim, table, max_pos));
    if (B * T == 0) return ok();
    if (!x || !w || !dy || !dx || !dw) return fail(DSC_ERR_NULL, "x, w, dy, dx and dw are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(dy) || !aligned16(dx) || !aligned16(dw))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const size_t wb = N * (D / H) * W * es;
    const Range in[] = {rng("x", x, N * D * es), rng("w", w, wb), rng("dy", dy, N * D * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0),
                        rng("table", table, rot ? (size_t)max_pos * head_dim * 4u : 0)};
    const Range out[] = {rng("dx", dx, N * D * es), rng("dw", dw, wb)};
    DSC_TRY(check_alias(in, 5, out, 2));
    dsc::HwProblem p{dt, B * T, T, D, W, H, x, w, dy, nullptr, dx, dw, cu_seqlens, n_seqs, residual,
                     rot, head_dim, table, max_pos};
    if (rot == 0) return launched(dsc::headwise_bwd(p, (hipStream_t)stream), "dsc_headwise_rope_bwd launch");
    return launched(dsc::headwise_rope_bwd(p, (hipStream_t)stream), "dsc_headwise_rope_bwd launch");
}

dsc_status dsc_lowrank_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                           int32_t R, const void *x, const void *z, const void *U,
                           const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *y) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (R < 1 || R > 128) return fail(DSC_ERR_SHAPE, "R = %d must be in 1..128", R);
    if (B * T == 0) return ok();  // empty batch: y has no elements
    if (!x || !z || !U || !y) return fail(DSC_ERR_NULL, "x, z, U and y are required");
    if (!aligned16(x) || !aligned16(z) || !aligned16(U) || !aligned16(y))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("z", z, N * R * es), rng("U", U, (size_t)R * D * W * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("y", y, N * D * es)};
    DSC_TRY(check_alias(in, 4, out, 1));
    dsc::LrProblem p{dt, B * T, T, D, W, R, x, z, U, nullptr, y, nullptr, nullptr, nullptr, nullptr,
                     cu_seqlens, n_seqs, residual};
    return launched(dsc::lowrank_fwd(p, (hipStream_t)stream), "dsc_lowrank_fwd launch");
}

dsc_status dsc_lowrank_rope_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                int32_t R, const void *x, const void *z, const void *U,
                                const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, int64_t rot,
                                int32_t head_dim, const float *table, int64_t max_pos, void *y) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (R < 1 || R > 128) return fail(DSC_ERR_SHAPE, "R = %d must be in 1..128", R);
    DSC_TRY(check_rope(dtype, B, T, D, cu_seqlens, rot, head_dim, table, max_pos));
    if (B * T == 0) return ok();
    if (!x || !z || !U || !y) return fail(DSC_ERR_NULL, "x, z, U and y are required");
    if (!aligned16(x) || !aligned16(z) || !aligned16(U) || !aligned16(y))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("z", z, N * R * es), rng("U", U, (size_t)R * D * W * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0),
                        rng("table", table, rot ? (size_t)max_pos * head_dim * 4u : 0)};
    const Range out[] = {rng("y", y, N * D * es)};
    DSC_TRY(check_alias(in, 5, out, 1));
    dsc::LrProblem p{dt, B * T, T, D, W, R, x, z, U, nullptr, y, nullptr, nullptr, nullptr, nullptr,
                     cu_seqlens, n_seqs, residual, rot, head_dim, table, max_pos};
    return launched(dsc::lowrank_rope_fwd(p, (hipStream_t)stream), "dsc_lowrank_rope_fwd launch");
}

namespace {

// Shape rules of the generated head-wise layer (both directions).
dsc_status check_gen(int dtype, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int64_t K,
                     const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (H < 1 || D % H) return fail(DSC_ERR_SHAPE, "H = %d must divide D = %lld", H, (long long)D);
    if (K < 1 || K > (1 << 20)) return fail(DSC_ERR_SHAPE, "K = %lld must be in 1..2^20", (long long)K);
    if (dtype != DSC_BF16) return fail(DSC_ERR_UNSUPPORTED, "the generated layer is implemented for DSC_BF16 only");
    if (K % 8) return fail(DSC_ERR_UNSUPPORTED, "K = %lld must be a multiple of 8", (long long)K);
    if ((D / H) * W % 8)
        return fail(DSC_ERR_UNSUPPORTED, "(D/H)*W = %lld must be a multiple of 8", (long long)((D / H) * W));
    return DSC_SUCCESS;
}


}  // namespace

dsc_status dsc_headwise_gen_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                                int64_t K, const void *h, const void *V, const void *x, const int32_t *cu_seqlens,
                                int32_t n_seqs, int32_t residual, void *y) {
    DSC_TRY(check_gen(dtype, B, T, D, W, H, K, cu_seqlens, n_seqs, residual));
    if (B * T == 0) return ok();
    if (!h || !V || !x || !y) return fail(DSC_ERR_NULL, "h, V, x and y are required");
    if (!aligned16(h) || !aligned16(V) || !aligned16(x) || !aligned16(y))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t N = (size_t)(B * T), GW = (size_t)((D / H) * W);
    const Range in[] = {rng("h", h, N * K * 2), rng("V", V, GW * K * 2), rng("x", x, N * D * 2),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("y", y, N * D * 2)};
    DSC_TRY(check_alias(in, 4, out, 1));
    dsc::GenProblem p{B * T, T, D, W, H, K, h, V, x, nullptr, y, nullptr, nullptr, nullptr, nullptr,
                      cu_seqlens, n_seqs, residual};
    return launched(dsc::headwise_gen_fwd(p, (hipStream_t)stream), "dsc_headwise_gen_fwd launch");
}

dsc_status dsc_generate_filters(void *stream, int dtype, int64_t N, int64_t K, int64_t C, const void *h,
                                const void *V, void *w) {
    if (dtype != DSC_BF16 && dtype != DSC_FP32) return fail(DSC_ERR_SHAPE, "dtype %d is not DSC_FP32 or DSC_BF16", dtype);
    if (N < 0 || K < 1 || K > (1 << 20) || C < 1 || C > (1 << 24))
        return fail(DSC_ERR_SHAPE, "N = %lld, K = %lld, C = %lld out of range", (long long)N, (long long)K,
                    (long long)C);
    if (dtype != DSC_BF16) return fail(DSC_ERR_UNSUPPORTED, "the filter generator is implemented for DSC_BF16 only");
    if (K % 8 || C % 8) return fail(DSC_ERR_UNSUPPORTED, "K and C must be multiples of 8");
    if (N == 0) return ok();
    if (!h || !V || !w) return fail(DSC_ERR_NULL, "h, V and w are required");
    if (!aligned16(h) || !aligned16(V) || !aligned16(w)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const Range in[] = {rng("h", h, (size_t)N * K * 2), rng("V", V, (size_t)C * K * 2)};
    const Range out[] = {rng("w", w, (size_t)N * C * 2)};
    DSC_TRY(check_alias(in, 2, out, 1));
    return launched(dsc::generate_filters(static_cast<const uint16_t *>(h), static_cast<const uint16_t *>(V), N, K, C,
                                          static_cast<uint16_t *>(w), (hipStream_t)stream),
                    "dsc_generate_filters launch");
}

size_t dsc_headwise_gen_bwd_workspace_size(int dtype, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                                           int64_t K) {
    if (check_gen(dtype, B, T, D, W, H, K, nullptr, 0, 0) != DSC_SUCCESS) return 0;
    return dsc::headwise_gen_bwd_workspace(B * T, D, W, H, K);
}

dsc_status dsc_headwise_gen_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                                int64_t K, const void *h, const void *V, const void *x, const void *dy,
                                const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *dx, void *dh,
                                float *dV, void *workspace, size_t workspace_bytes) {
    DSC_TRY(check_gen(dtype, B, T, D, W, H, K, cu_seqlens, n_seqs, residual));
    const size_t GW = (size_t)((D / H) * W);
    if (B * T == 0) {  // dV is a sum over no tokens: zero
        if (!dV) return fail(DSC_ERR_NULL, "dV is required");
        if (!aligned16(dV)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
        return launched(dsc::lowrank_zero(dV, (int64_t)(GW * K), (hipStream_t)stream), "dsc_headwise_gen_bwd launch");
    }
    if (!h || !V || !x || !dy || !dx || !dh || !dV) return fail(DSC_ERR_NULL, "h, V, x, dy, dx, dh and dV are required");
    if (!aligned16(h) || !aligned16(V) || !aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(dh) ||
        !aligned16(dV))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t N = (size_t)(B * T), need = dsc::headwise_gen_bwd_workspace(B * T, D, W, H, K);
    if (!workspace || workspace_bytes < need)
        return fail(DSC_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(DSC_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    const Range in[] = {rng("h", h, N * K * 2), rng("V", V, GW * K * 2), rng("x", x, N * D * 2),
                        rng("dy", dy, N * D * 2), rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("dx", dx, N * D * 2), rng("dh", dh, N * K * 2), rng("dV", dV, GW * K * 4),
                         rng("workspace", workspace, need)};
    DSC_TRY(check_alias(in, 5, out, 4));
    dsc::GenProblem p{B * T, T, D, W, H, K, h, V, x, dy, nullptr, dx, dh, dV, workspace, cu_seqlens, n_seqs,
                      residual};
    return launched(dsc::headwise_gen_bwd(p, (hipStream_t)stream), "dsc_headwise_gen_bwd launch");
}

size_t dsc_lowrank_bwd_workspace_size(int dtype, int64_t B, int64_t T, int64_t D, int32_t W, int32_t R) {
    if (check_common(dtype, B, T, D, W, nullptr, 0, 0) != DSC_SUCCESS || R < 1 || R > 128) return 0;
    return dsc::lowrank_bwd_workspace(dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32, B * T, D, W, R);
}

namespace {

// The rotary embedding that follows the layer (dsc_lowrank_rope_bwd).
struct RopeArgs {
    int64_t rot;
    int32_t head_dim;
    const float *table;
    int64_t max_pos;
};

// Validation and launch shared by the low-rank backward entry points.
// noalloc: no workspace argument; the accumulator is the device's built-in
// scratch, whose address is taken only after every other check passed.
// rope: the layer followed by the rotary embedding (the fused backward, never
// the split one, so its workspace is at most dsc_lowrank_bwd_workspace_size).
dsc_status lowrank_bwd_call(bool det, const char *name, void *stream, int dtype, int64_t B, int64_t T, int64_t D,
                            int32_t W, int32_t R, const void *x, const void *z, const void *U, const void *dy,
                            const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *dx, void *dz,
                            float *dU, void *workspace, size_t workspace_bytes, bool noalloc = false,
                            const RopeArgs *rope = nullptr) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (R < 1 || R > 128) return fail(DSC_ERR_SHAPE, "R = %d must be in 1..128", R);
    if (rope) DSC_TRY(check_rope(dtype, B, T, D, cu_seqlens, rope->rot, rope->head_dim, rope->table, rope->max_pos));
    if (B * T == 0) {  // empty batch: dU is a sum over no tokens, zero; nothing else has elements
        if (!dU) return fail(DSC_ERR_NULL, "dU is required");
        if (!aligned16(dU)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
        return launched(dsc::lowrank_zero(dU, (int64_t)R * D * W, (hipStream_t)stream), name);
    }
    if (!x || !z || !U || !dy || !dx || !dz || !dU)
        return fail(DSC_ERR_NULL, "x, z, U, dy, dx, dz and dU are required");
    if (!aligned16(x) || !aligned16(z) || !aligned16(U) || !aligned16(dy) || !aligned16(dx) ||
        !aligned16(dz) || !aligned16(dU))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    const size_t need = det ? dsc::lowrank_bwd_det_workspace(dt, B * T, D, W, R)
                            : dsc::lowrank_bwd_workspace(dt, B * T, D, W, R, !noalloc && !rope);
    if (noalloc) {
        if (need > (size_t)dsc::kNoallocScratchFloats * sizeof(float))
            return fail(DSC_ERR_WORKSPACE,
                        "B*T*R = %lld exceeds the built-in scratch of %lld fp32 values (use dsc_lowrank_bwd "
                        "with a workspace)",
                        (long long)(B * T * R), (long long)dsc::kNoallocScratchFloats);
    } else if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(DSC_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(DSC_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    }
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("z", z, N * R * es), rng("U", U, (size_t)R * D * W * es),
                        rng("dy", dy, N * D * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0),
                        rng("table", rope ? rope->table : nullptr,
                            rope && rope->rot ? (size_t)rope->max_pos * rope->head_dim * 4u : 0)};
    const Range out[] = {rng("dx", dx, N * D * es), rng("dz", dz, N * R * es),
                         rng("dU", dU, (size_t)R * D * W * 4),
                         rng("workspace", workspace, need && !noalloc ? need : 0)};
    DSC_TRY(check_alias(in, 6, out, 4));
    if (noalloc && need > 0) {
        float *scratch = nullptr;
        const hipError_t e = dsc::noalloc_scratch(&scratch);
        if (e != hipSuccess) return fail(DSC_ERR_HIP, "%s: scratch address: %s", name, hipGetErrorString(e));
        workspace = scratch;
    }
    float *acc = need ? static_cast<float *>(workspace) : det ? nullptr : static_cast<float *>(dz);
    dsc::LrProblem p{dt, B * T, T, D, W, R, x, z, U, dy, nullptr, dx, dz, dU, acc, cu_seqlens, n_seqs, residual};
    if (rope) {
        p.rot = rope->rot;
        p.hd = rope->head_dim;
        p.rope = rope->table;
        p.max_pos = rope->max_pos;
        return launched(dsc::lowrank_rope_bwd(p, (hipStream_t)stream), name);
    }
    return launched(det ? dsc::lowrank_bwd_det(p, (hipStream_t)stream)
                        : dsc::lowrank_bwd(p, (hipStream_t)stream, !noalloc),
                    name);
}

}  // namespace

dsc_status dsc_lowrank_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                           int32_t R, const void *x, const void *z, const void *U, const void *dy,
                           const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *dx,
                           void *dz, float *dU, void *workspace, size_t workspace_bytes) {
    return lowrank_bwd_call(false, "dsc_lowrank_bwd launch", stream, dtype, B, T, D, W, R, x, z, U, dy, cu_seqlens,
                            n_seqs, residual, dx, dz, dU, workspace, workspace_bytes);
}

dsc_status dsc_lowrank_rope_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                int32_t R, const void *x, const void *z, const void *U, const void *dy,
                                const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, int64_t rot,
                                int32_t head_dim, const float *table, int64_t max_pos, void *dx, void *dz,
                                float *dU, void *workspace, size_t workspace_bytes) {
    const RopeArgs rope{rot, head_dim, table, max_pos};
    return lowrank_bwd_call(false, "dsc_lowrank_rope_bwd launch", stream, dtype, B, T, D, W, R, x, z, U, dy,
                            cu_seqlens, n_seqs, residual, dx, dz, dU, workspace, workspace_bytes, false, &rope);
}

dsc_status dsc_lowrank_bwd_noalloc(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                   int32_t R, const void *x, const void *z, const void *U, const void *dy,
                                   const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *dx,
                                   void *dz, float *dU) {
    return lowrank_bwd_call(false, "dsc_lowrank_bwd_noalloc launch", stream, dtype, B, T, D, W, R, x, z, U, dy,
                            cu_seqlens, n_seqs, residual, dx, dz, dU, nullptr, 0, true);
}

size_t dsc_lowrank_bwd_deterministic_workspace_size(int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                                    int32_t R) {
    if (check_common(dtype, B, T, D, W, nullptr, 0, 0) != DSC_SUCCESS || R < 1 || R > 128) return 0;
    return dsc::lowrank_bwd_det_workspace(dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32, B * T, D, W, R);
}

dsc_status dsc_lowrank_bwd_deterministic(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                         int32_t R, const void *x, const void *z, const void *U, const void *dy,
                                         const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual, void *dx,
                                         void *dz, float *dU, void *workspace, size_t workspace_bytes) {
    return lowrank_bwd_call(true, "dsc_lowrank_bwd_deterministic launch", stream, dtype, B, T, D, W, R, x, z, U, dy,
                            cu_seqlens, n_seqs, residual, dx, dz, dU, workspace, workspace_bytes);
}

dsc_status dsc_static_fwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                          const void *x, const void *c, const int32_t *cu_seqlens, int32_t n_seqs,
                          int32_t residual, void *y) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    if (B * T == 0) return ok();  // empty batch: y has no elements
    if (!x || !c || !y) return fail(DSC_ERR_NULL, "x, c and y are required");
    if (!aligned16(x) || !aligned16(c) || !aligned16(y)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("c", c, (size_t)D * W * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("y", y, N * D * es)};
    DSC_TRY(check_alias(in, 3, out, 1));
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    dsc::StProblem p{dt, B * T, T, D, W, x, c, nullptr, y, nullptr, nullptr, cu_seqlens, n_seqs, residual};
    return launched(dsc::static_fwd(p, (hipStream_t)stream), "dsc_static_fwd launch");
}

namespace {

// Validation and launch shared by the two static backward entry points.
dsc_status static_bwd_call(bool det, const char *name, void *stream, int dtype, int64_t B, int64_t T, int64_t D,
                           int32_t W, const void *x, const void *c, const void *dy, const int32_t *cu_seqlens,
                           int32_t n_seqs, int32_t residual, void *dx, float *dc, void *workspace,
                           size_t workspace_bytes) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, residual));
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    if (B * T == 0) {  // empty batch: dc is a sum over no tokens, zero; dx has no elements
        if (!dc) return fail(DSC_ERR_NULL, "dc is required");
        if (!aligned16(dc)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
        dsc::StProblem p{dt, 0, T, D, W, nullptr, nullptr, nullptr, nullptr, nullptr, dc, nullptr, 0, residual};
        return launched(dsc::static_bwd(p, (hipStream_t)stream), name);
    }
    if (!x || !c || !dy || !dx || !dc) return fail(DSC_ERR_NULL, "x, c, dy, dx and dc are required");
    if (!aligned16(x) || !aligned16(c) || !aligned16(dy) || !aligned16(dx) || !aligned16(dc))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t need = det ? dsc::static_bwd_det_workspace(dt, B * T, D, W) : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(DSC_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(DSC_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    }
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const Range in[] = {rng("x", x, N * D * es), rng("c", c, (size_t)D * W * es), rng("dy", dy, N * D * es),
                        rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("dx", dx, N * D * es), rng("dc", dc, (size_t)D * W * 4),
                         rng("workspace", workspace, need)};
    DSC_TRY(check_alias(in, 4, out, 3));
    dsc::StProblem p{dt, B * T, T, D, W, x, c, dy, nullptr, dx, dc, cu_seqlens, n_seqs, residual};
    const hipError_t e = det ? dsc::static_bwd_det(p, static_cast<float *>(workspace), (hipStream_t)stream)
                             : dsc::static_bwd(p, (hipStream_t)stream);
    return launched(e, name);
}

}  // namespace

dsc_status dsc_static_bwd(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                          const void *x, const void *c, const void *dy, const int32_t *cu_seqlens,
                          int32_t n_seqs, int32_t residual, void *dx, float *dc) {
    return static_bwd_call(false, "dsc_static_bwd launch", stream, dtype, B, T, D, W, x, c, dy, cu_seqlens, n_seqs,
                           residual, dx, dc, nullptr, 0);
}

size_t dsc_static_bwd_deterministic_workspace_size(int dtype, int64_t B, int64_t T, int64_t D, int32_t W) {
    if (check_common(dtype, B, T, D, W, nullptr, 0, 0) != DSC_SUCCESS) return 0;
    return dsc::static_bwd_det_workspace(dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32, B * T, D, W);
}

dsc_status dsc_static_bwd_deterministic(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                        const void *x, const void *c, const void *dy, const int32_t *cu_seqlens,
                                        int32_t n_seqs, int32_t residual, void *dx, float *dc, void *workspace,
                                        size_t workspace_bytes) {
    return static_bwd_call(true, "dsc_static_bwd_deterministic launch", stream, dtype, B, T, D, W, x, c, dy,
                           cu_seqlens, n_seqs, residual, dx, dc, workspace, workspace_bytes);
}

namespace {

// Shared checks of the two decoding steps (B sequences, one token each).
dsc_status check_decode(int dtype, int64_t B, int64_t D, int32_t W, int32_t residual) {
    if (dtype != DSC_FP32 && dtype != DSC_BF16) return fail(DSC_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (B < 0 || D < 1 || D > ((int64_t)1 << 24) || B > (int64_t)INT32_MAX / D)  // B*D < 2^31, no product formed
        return fail(DSC_ERR_SHAPE, "B >= 0, D in 1..2^24 and B*D < 2^31 required (got %lld, %lld)", (long long)B,
                    (long long)D);
    if (W < 1 || W > 8) return fail(DSC_ERR_SHAPE, "W must be in 1..8 (got %d)", W);
    const int vec = dtype == DSC_BF16 ? 8 : 4;
    if (D % vec) return fail(DSC_ERR_SHAPE, "D = %lld must be a multiple of %d for this dtype", (long long)D, vec);
    if (residual != 0 && residual != 1) return fail(DSC_ERR_SHAPE, "residual must be 0 or 1");
    return DSC_SUCCESS;
}

}  // namespace

namespace {

// The head-wise decoding step, with the rotation of y when rot > 0.
dsc_status headwise_decode_call(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t H,
                                const void *x, const void *w, void *state, int32_t residual, void *y, int64_t rot,
                                int32_t head_dim, const float *table, int64_t max_pos, const int32_t *positions,
                                const char *what) {
    DSC_TRY(check_decode(dtype, B, D, W, residual));
    if (H < 1 || D % H) return fail(DSC_ERR_SHAPE, "H = %d must divide D = %lld", H, (long long)D);
    const int vec = dtype == DSC_BF16 ? 8 : 4;
    if (rot != 0 || head_dim != 0) {
        if (head_dim < 2 || head_dim % 2 || head_dim > (1 << 16))
            return fail(DSC_ERR_SHAPE, "head_dim = %d must be even, in 2..65536", head_dim);
        if (head_dim % vec)
            return fail(DSC_ERR_UNSUPPORTED, "head_dim = %d must be a multiple of %d for this dtype", head_dim, vec);
        if (rot < 0 || rot > D || rot % head_dim)
            return fail(DSC_ERR_SHAPE, "rot = %lld must be a multiple of head_dim in 0..D", (long long)rot);
    }
    if (B == 0) return ok();
    if (!x || !w || !y || (W > 1 && !state)) return fail(DSC_ERR_NULL, "x, w, y and (W > 1) state are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned16(state))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    if (rot > 0) {
        if (!table || !positions) return fail(DSC_ERR_NULL, "table and positions are required when rot > 0");
        if (!aligned16(table) || ((uintptr_t)positions & 3u))
            return fail(DSC_ERR_ALIGNMENT, "table must be 16-byte and positions 4-byte aligned");
        if (max_pos < 1 || max_pos > INT32_MAX / head_dim)
            return fail(DSC_ERR_SHAPE, "max_pos = %lld out of range", (long long)max_pos);
    }
    const size_t es = esize(dtype), Bs = (size_t)B;
    const Range in[] = {rng("x", x, Bs * D * es), rng("w", w, Bs * (D / H) * W * es),
                        rng("table", table, rot > 0 ? (size_t)max_pos * head_dim * 4u : 0),
                        rng("positions", positions, rot > 0 ? Bs * 4u : 0)};
    const Range out[] = {rng("y", y, Bs * D * es), rng("state", state, W > 1 ? Bs * (W - 1) * D * es : 0)};
    DSC_TRY(check_alias(in, 4, out, 2));
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    dsc::DecProblem p{dt, B, D, W, H, 0, false, x, w, nullptr, nullptr, state, y, residual,
                      rot, head_dim, table, max_pos, positions};
    return launched(dsc::decode_step(p, (hipStream_t)stream), what);
}

}  // namespace

dsc_status dsc_headwise_decode(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t H,
                               const void *x, const void *w, void *state, int32_t residual, void *y) {
    return headwise_decode_call(stream, dtype, B, D, W, H, x, w, state, residual, y, 0, 0, nullptr, 0, nullptr,
                                "dsc_headwise_decode launch");
}

dsc_status dsc_headwise_rope_decode(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t H,
                                    const void *x, const void *w, void *state, int32_t residual, int64_t rot,
                                    int32_t head_dim, const float *table, int64_t max_pos,
                                    const int32_t *positions, void *y) {
    if (rot == 0 && head_dim == 0) return fail(DSC_ERR_SHAPE, "head_dim is required");
    return headwise_decode_call(stream, dtype, B, D, W, H, x, w, state, residual, y, rot, head_dim, table, max_pos,
                                positions, "dsc_headwise_rope_decode launch");
}

dsc_status dsc_lowrank_decode(void *stream, int dtype, int64_t B, int64_t D, int32_t W, int32_t R,
                              const void *x, const void *z, const void *U, void *state, int32_t residual,
                              void *y) {
    DSC_TRY(check_decode(dtype, B, D, W, residual));
    if (R < 1 || R > 128) return fail(DSC_ERR_SHAPE, "R = %d must be in 1..128", R);
    if (B == 0) return ok();
    if (!x || !z || !U || !y || (W > 1 && !state))
        return fail(DSC_ERR_NULL, "x, z, U, y and (W > 1) state are required");
    if (!aligned16(x) || !aligned16(z) || !aligned16(U) || !aligned16(y) || !aligned16(state))
        return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), Bs = (size_t)B;
    const Range in[] = {rng("x", x, Bs * D * es), rng("z", z, Bs * R * es), rng("U", U, (size_t)R * D * W * es)};
    const Range out[] = {rng("y", y, Bs * D * es), rng("state", state, W > 1 ? Bs * (W - 1) * D * es : 0)};
    DSC_TRY(check_alias(in, 3, out, 2));
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    dsc::DecProblem p{dt, B, D, W, 0, R, true, x, nullptr, z, U, state, y, residual};
    return launched(dsc::decode_step(p, (hipStream_t)stream), "dsc_lowrank_decode launch");
}

dsc_status dsc_state_from_prefill(void *stream, int dtype, int64_t B, int64_t T, int64_t D, int32_t W,
                                  const void *x, const int32_t *cu_seqlens, int32_t n_seqs, void *state) {
    DSC_TRY(check_common(dtype, B, T, D, W, cu_seqlens, n_seqs, 0));
    if (B * T == 0 || W == 1) return ok();  // no sequences, or a state without slots
    if (!x || !state) return fail(DSC_ERR_NULL, "x and state are required");
    if (!aligned16(x) || !aligned16(state)) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t es = esize(dtype), N = (size_t)(B * T);
    const size_t nseq = cu_seqlens ? (size_t)n_seqs : (size_t)B;
    const Range in[] = {rng("x", x, N * D * es), rng("cu_seqlens", cu_seqlens, cu_seqlens ? 4u * (n_seqs + 1) : 0)};
    const Range out[] = {rng("state", state, nseq * (W - 1) * D * es)};
    DSC_TRY(check_alias(in, 2, out, 1));
    const dsc::Dtype dt = dtype == DSC_BF16 ? dsc::Dtype::BF16 : dsc::Dtype::F32;
    return launched(dsc::state_from_prefill(dt, x, cu_seqlens, n_seqs, B, T, D, W, state, (hipStream_t)stream),
                    "dsc_state_from_prefill launch");
}

dsc_status dsc_bench_stream(void *stream, const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                            int32_t unroll, int32_t load_nt, int32_t store_nt, int32_t chunked, int64_t blocks) {
    const int64_t kMax = (int64_t)1 << 40;
    if (read_bytes < 0 || write_bytes < 0 || read_bytes >= kMax || write_bytes >= kMax || read_bytes % 16 ||
        write_bytes % 16)
        return fail(DSC_ERR_SHAPE, "byte counts must be multiples of 16 in [0, 2^40)");
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8)
        return fail(DSC_ERR_SHAPE, "unroll must be 1, 2, 4 or 8 (got %d)", unroll);
    if ((load_nt != 0 && load_nt != 1) || (store_nt != 0 && store_nt != 1) || (chunked != 0 && chunked != 1))
        return fail(DSC_ERR_SHAPE, "load_nt, store_nt and chunked must be 0 or 1");
    if (blocks < 0 || blocks > ((int64_t)1 << 30)) return fail(DSC_ERR_SHAPE, "blocks out of range");
    if (!dst || (read_bytes && !src)) return fail(DSC_ERR_NULL, "dst (and src when reading) are required");
    if (!aligned16(dst) || (src && !aligned16(src))) return fail(DSC_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const Range in[] = {rng("src", src, (size_t)read_bytes)};
    const Range out[] = {rng("dst", dst, (size_t)(write_bytes > 16 ? write_bytes : 16))};
    DSC_TRY(check_alias(in, 1, out, 1));
    return launched(dsc::stream_probe(src, read_bytes, dst, write_bytes, unroll, load_nt == 1, store_nt == 1,
                                      chunked == 1, blocks, (hipStream_t)stream),
                    "dsc_bench_stream launch");
}

const char *dsc_status_string(int status) {
    switch (status) {
        case DSC_SUCCESS: return "DSC_SUCCESS";
        case DSC_ERR_NULL: return "DSC_ERR_NULL";
        case DSC_ERR_SHAPE: return "DSC_ERR_SHAPE";
        case DSC_ERR_UNSUPPORTED: return "DSC_ERR_UNSUPPORTED";
        case DSC_ERR_ALIGNMENT: return "DSC_ERR_ALIGNMENT";
        case DSC_ERR_ALIAS: return "DSC_ERR_ALIAS";
        case DSC_ERR_WORKSPACE: return "DSC_ERR_WORKSPACE";
        case DSC_ERR_HIP: return "DSC_ERR_HIP";
        default: return "DSC_UNKNOWN_STATUS";
    }
}

const char *dsc_last_error(void) { return g_last_error; }

int dsc_abi_version(void) { return DSC_ABI_VERSION; }

}  // extern "C"
