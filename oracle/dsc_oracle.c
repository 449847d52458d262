/*
 * dsc_oracle.c -- plain, slow, fp64 CPU reference of the dynamic short
 * convolution (forward and backward, head-wise tied and low-rank filters).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source, header, table or helper
 * with the HIP library.
 *
 * Source of the definitions ("Dynamic Short Convolutions Improve
 * Transformers", the gist.science technical summaries, es/fr/de/hi):
 *   - Methodology, "mechanism": for activations x_t the output is the sum
 *     over taps k = 0..W-1 of w(t)_k (elementwise) x_{t-k}; the filter w(t)
 *     depends on the token t.
 *   - Methodology, "parametrization": (1) low-rank factorisation of rank R,
 *     read as w(t) = z_t U with U of shape (R, D*W); (2) head-wise tying,
 *     one filter shared by H consecutive channels.
 *   - Methodology, "placement": residual form X = X + dynamicShortConv(X).
 * and the authors' thread ("Custom Triton GPU kernels maintain wall-clock
 * training efficiency", digg.com): the static short convolution being
 * generalised is depthwise and causal, so x before a sequence start is zero.
 * That static layer itself (one filter per channel, the same at every
 * position) is the next pair of functions below, followed by the decoding
 * step and, last, the rotary position embedding that the placement puts
 * right after the layer on the query and key projections.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - tap k = 0 multiplies the current token x_t;
 *   - x_{t-k} is zero when t-k lies before the first token of t's segment
 *     (zero left padding per sequence; packed sequences reset causally);
 *   - channel d uses head-wise filter j = floor(d / H);
 *   - w has layout (B,T,D/H,W), tap innermost; U is (R, D*W) read as
 *     (R, D, W), i.e. column d*W + k;
 *   - no nonlinearity, normalisation or bias is applied to w.
 * The backward pass is the chain rule of the forward definition for
 * L = <dy, y>; it is written out directly below.
 *
 * Every value is held and accumulated in double.  OpenMP parallelises over
 * output rows (or dU columns); each output element is a sequential sum in a
 * fixed order, so results do not depend on the thread count.
 *
 * All functions return 0 on success, -1 on allocation failure and -2 on an
 * invalid argument.  Row outputs cover tokens [n_lo, n_hi) only and are
 * stored compactly (row n goes to row n - n_lo of the output); dU covers
 * channels [d_lo, d_hi) only, stored as (R, (d_hi-d_lo)*W).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI_VERSION 1

int oracle_abi_version(void) { return ORACLE_ABI_VERSION; }

/* Threads an OpenMP loop of the oracle runs with. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* First token of the segment of every flattened token n in [0, B*T).
 * Without cu_seqlens each of the B rows is one sequence; otherwise
 * cu_seqlens[0..n_seqs] are increasing offsets from 0 to B*T. */
static int64_t *segment_starts(int64_t B, int64_t T, const int32_t *cu_seqlens, int32_t n_seqs)
{
    int64_t N = B * T;
    int64_t *seg = (int64_t *)malloc((size_t)(N > 0 ? N : 1) * sizeof *seg);
    if (!seg) return NULL;
    if (cu_seqlens == NULL || n_seqs == 0) {
        for (int64_t n = 0; n < N; ++n) seg[n] = (n / T) * T;
    } else {
        for (int32_t i = 0; i < n_seqs; ++i)
            for (int64_t n = cu_seqlens[i]; n < cu_seqlens[i + 1]; ++n) seg[n] = cu_seqlens[i];
    }
    return seg;
}

static int check_common(int64_t B, int64_t T, int64_t D, int32_t W, const int32_t *cu, int32_t n_seqs,
                        int64_t n_lo, int64_t n_hi)
{
    if (B < 1 || T < 1 || D < 1 || W < 1) return -2;
    if (n_lo < 0 || n_hi < n_lo || n_hi > B * T) return -2;
    if (cu != NULL && n_seqs > 0) {
        if (cu[0] != 0 || cu[n_seqs] != B * T) return -2;
        for (int32_t i = 0; i < n_seqs; ++i)
            if (cu[i + 1] <= cu[i]) return -2;
    }
    return 0;
}

/* ---------------------------------------------------------------- head-wise */

/* y[n,d] = rho*x[n,d] + sum_{k<W, n-k >= seg(n)} w[n, d/H, k] * x[n-k, d] */
int oracle_headwise_fwd(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                        const double *x, const double *w,
                        const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                        int64_t n_lo, int64_t n_hi, double *y)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, n_lo, n_hi) || H < 1 || D % H) return -2;
    const int64_t G = D / H;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = n_lo; n < n_hi; ++n) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? x[n * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k)
                if (n - k >= seg[n]) acc += w[(n * G + d / H) * W + k] * x[(n - k) * D + d];
            y[(n - n_lo) * D + d] = acc;
        }
    }
    free(seg);
    return 0;
}

/* Chain rule of the forward for L = <g, y>:
 *   dx[m,d]   = rho*g[m,d] + sum_{k: m+k < N, m >= seg(m+k)} w[m+k, d/H, k] * g[m+k, d]
 *   dw[n,j,k] = [n-k >= seg(n)] * sum_{d = jH .. jH+H-1} g[n,d] * x[n-k,d]          */
int oracle_headwise_bwd(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H,
                        const double *x, const double *w, const double *g,
                        const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                        int64_t n_lo, int64_t n_hi, double *dx, double *dw)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, n_lo, n_hi) || H < 1 || D % H) return -2;
    const int64_t N = B * T, G = D / H;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = n_lo; m < n_hi; ++m) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? g[m * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k) {
                int64_t n = m + k;
                if (n < N && m >= seg[n]) acc += w[(n * G + d / H) * W + k] * g[n * D + d];
            }
            dx[(m - n_lo) * D + d] = acc;
        }
        for (int64_t j = 0; j < G; ++j) {
            for (int32_t k = 0; k < W; ++k) {
                double acc = 0.0;
                if (m - k >= seg[m])
                    for (int64_t d = j * H; d < (j + 1) * H; ++d) acc += g[m * D + d] * x[(m - k) * D + d];
                dw[((m - n_lo) * G + j) * W + k] = acc;
            }
        }
    }
    free(seg);
    return 0;
}

/* ----------------------------------------------------------------- low-rank */

/* Filter of token n, channel d, tap k: w[n,d,k] = sum_r z[n,r] * U[r, d*W+k]. */
static double lowrank_filter(int64_t D, int32_t W, int32_t R, const double *z, const double *U,
                             int64_t n, int64_t d, int32_t k)
{
    double acc = 0.0;
    for (int32_t r = 0; r < R; ++r) acc += z[n * R + r] * U[(int64_t)r * D * W + d * W + k];
    return acc;
}

/* y[n,d] = rho*x[n,d] + sum_{k<W, n-k >= seg(n)} w[n,d,k] * x[n-k,d], w from z and U */
int oracle_lowrank_fwd(int64_t B, int64_t T, int64_t D, int32_t W, int32_t R,
                       const double *x, const double *z, const double *U,
                       const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                       int64_t n_lo, int64_t n_hi, double *y)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, n_lo, n_hi) || R < 1) return -2;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = n_lo; n < n_hi; ++n) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? x[n * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k)
                if (n - k >= seg[n]) acc += lowrank_filter(D, W, R, z, U, n, d, k) * x[(n - k) * D + d];
            y[(n - n_lo) * D + d] = acc;
        }
    }
    free(seg);
    return 0;
}

/* Chain rule for L = <g, y> with w = zU and the per-channel filter gradient
 *   dwc[n,d,k] = [n-k >= seg(n)] * g[n,d] * x[n-k,d]:
 *   dx[m,d]        = rho*g[m,d] + sum_{k: m+k < N, m >= seg(m+k)} w[m+k,d,k] * g[m+k,d]
 *   dz[n,r]        = sum_{d,k} U[r, d*W+k] * dwc[n,d,k]
 *   dU[r, d*W+k]   = sum_n z[n,r] * dwc[n,d,k]                                      */
int oracle_lowrank_bwd(int64_t B, int64_t T, int64_t D, int32_t W, int32_t R,
                       const double *x, const double *z, const double *U, const double *g,
                       const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                       int64_t n_lo, int64_t n_hi, double *dx, double *dz,
                       int64_t d_lo, int64_t d_hi, double *dU)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, n_lo, n_hi) || R < 1) return -2;
    if (d_lo < 0 || d_hi < d_lo || d_hi > D) return -2;
    const int64_t N = B * T;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;

#pragma omp parallel for schedule(static)
    for (int64_t m = n_lo; m < n_hi; ++m) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? g[m * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k) {
                int64_t n = m + k;
                if (n < N && m >= seg[n]) acc += lowrank_filter(D, W, R, z, U, n, d, k) * g[n * D + d];
            }
            dx[(m - n_lo) * D + d] = acc;
        }
        for (int32_t r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d)
                for (int32_t k = 0; k < W; ++k)
                    if (m - k >= seg[m])
                        acc += U[(int64_t)r * D * W + d * W + k] * (g[m * D + d] * x[(m - k) * D + d]);
            dz[(m - n_lo) * R + r] = acc;
        }
    }

    const int64_t DWs = (d_hi - d_lo) * W;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < DWs; ++c) {
        const int64_t d = d_lo + c / W;
        const int32_t k = (int32_t)(c % W);
        for (int32_t r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n)
                if (n - k >= seg[n]) acc += z[n * R + r] * (g[n * D + d] * x[(n - k) * D + d]);
            dU[(int64_t)r * DWs + c] = acc;
        }
    }
    free(seg);
    return 0;
}

/* ------------------------------------------------------------ static filter */

/* The fixed-filter layer that the dynamic convolution generalises (authors'
 * thread on digg.com: a depthwise causal convolution of small width, the
 * same filter at every position), with tap k weighting lag k as above:
 *   y[n,d] = rho*x[n,d] + sum_{k<W, n-k >= seg(n)} c[d,k] * x[n-k,d]
 * c has layout (D, W), tap innermost.                                        */
int oracle_static_fwd(int64_t B, int64_t T, int64_t D, int32_t W, const double *x, const double *c,
                      const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                      int64_t n_lo, int64_t n_hi, double *y)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, n_lo, n_hi)) return -2;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = n_lo; n < n_hi; ++n) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? x[n * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k)
                if (n - k >= seg[n]) acc += c[d * W + k] * x[(n - k) * D + d];
            y[(n - n_lo) * D + d] = acc;
        }
    }
    free(seg);
    return 0;
}

/* Chain rule for L = <g, y>:
 *   dx[m,d] = rho*g[m,d] + sum_{k: m+k < N, m >= seg(m+k)} c[d,k] * g[m+k,d]
 *   dc[d,k] = sum over every token n of [n-k >= seg(n)] * g[n,d] * x[n-k,d]
 * dx covers tokens [n_lo, n_hi); dc is (D, W) over all tokens.               */
int oracle_static_bwd(int64_t B, int64_t T, int64_t D, int32_t W, const double *x, const double *c,
                      const double *g, const int32_t *cu_seqlens, int32_t n_seqs, int32_t residual,
                      int64_t n_lo, int64_t n_hi, double *dx, double *dc)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, n_lo, n_hi)) return -2;
    const int64_t N = B * T;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = n_lo; m < n_hi; ++m) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? g[m * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k) {
                int64_t n = m + k;
                if (n < N && m >= seg[n]) acc += c[d * W + k] * g[n * D + d];
            }
            dx[(m - n_lo) * D + d] = acc;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < D * W; ++i) {
        const int64_t d = i / W;
        const int32_t k = (int32_t)(i % W);
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n)
            if (n - k >= seg[n]) acc += g[n * D + d] * x[(n - k) * D + d];
        dc[i] = acc;
    }
    free(seg);
    return 0;
}

/* ---------------------------------------------------------- filter generator */

/* The head-wise filters as a learned linear map of the current hidden state
 * ("Dynamic Short Convolutions Improve Transformers", gist.science technical
 * summary, Methodology: parametrization), written as a linear layer with
 * weight V (C, K): for rows n in [n_lo, n_hi) of h (N, K),
 *   w[n, c] = sum_{j<K} h[n, j] * V[c, j],   c = g*W + k  (C = G*W).
 * w is stored compactly (row n at n - n_lo).                                */
int oracle_generate(int64_t N, int64_t K, int64_t C, const double *h, const double *V, int64_t n_lo,
                    int64_t n_hi, double *w)
{
    if (N < 0 || K < 1 || C < 1 || n_lo < 0 || n_hi > N || n_lo > n_hi) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t n = n_lo; n < n_hi; ++n)
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < K; ++j) acc += h[n * K + j] * V[c * K + j];
            w[(n - n_lo) * C + c] = acc;
        }
    return 0;
}

/* Chain rule of the map for L = <dw, w>:
 *   dh[n, j] = sum_{c<C} dw[n, c] * V[c, j]   for rows [n_lo, n_hi) (dw and dh
 *              stored compactly, row n at n - n_lo),
 *   dV[c, j] = sum_{n<N} dw[n, c] * h[n, j]   for c in [c_lo, c_hi) (dw (N, C)
 *              over every row; dV row c at c - c_lo).                       */
int oracle_generate_bwd_h(int64_t K, int64_t C, const double *dw, const double *V, int64_t rows, double *dh)
{
    if (K < 1 || C < 1 || rows < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t j = 0; j < K; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < C; ++c) acc += dw[n * C + c] * V[c * K + j];
            dh[n * K + j] = acc;
        }
    return 0;
}

int oracle_generate_bwd_v(int64_t N, int64_t K, int64_t C, const double *dw, const double *h, int64_t c_lo,
                          int64_t c_hi, double *dV)
{
    if (N < 0 || K < 1 || C < 1 || c_lo < 0 || c_hi > C || c_lo > c_hi) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t c = c_lo; c < c_hi; ++c)
        for (int64_t j = 0; j < K; ++j) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += dw[n * C + c] * h[n * K + j];
            dV[(c - c_lo) * K + j] = acc;
        }
    return 0;
}

/* ---------------------------------------------------------------- decoding */

/* One token per sequence at inference (the pages' inference remark: decoding
 * needs its own path).  Sequence b carries a state of its last W-1 inputs,
 * state[b, i, d] = x of its token t-1-i (i = 0 the most recent), zero for
 * positions before the sequence's first token.  For the new token x[b, d]:
 *   y[b,d] = rho*x[b,d] + w[b,j,0]*x[b,d] + sum_{k=1}^{W-1} w[b,j,k]*state[b,k-1,d]
 * with j = d/H (head-wise; w is (B, D/H, W)), which is the forward of the
 * sequence evaluated at its newest token.  The state then shifts:
 *   state'[b,0,d] = x[b,d],  state'[b,i,d] = state[b,i-1,d] (i >= 1).
 * state (B, W-1, D) is read and overwritten; y is (B, D).                  */
int oracle_headwise_decode(int64_t B, int64_t D, int32_t W, int32_t H, const double *x, const double *w,
                           double *state, int32_t residual, double *y)
{
    if (B < 1 || D < 1 || W < 1 || H < 1 || D % H) return -2;
    const int64_t G = D / H;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? x[b * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k) {
                double xv = k == 0 ? x[b * D + d] : state[(b * (W - 1) + (k - 1)) * D + d];
                acc += w[(b * G + d / H) * W + k] * xv;
            }
            y[b * D + d] = acc;
        }
        for (int32_t i = W - 2; i >= 1; --i)
            for (int64_t d = 0; d < D; ++d)
                state[(b * (W - 1) + i) * D + d] = state[(b * (W - 1) + i - 1) * D + d];
        if (W > 1)
            for (int64_t d = 0; d < D; ++d) state[(b * (W - 1)) * D + d] = x[b * D + d];
    }
    return 0;
}

/* Low-rank decode: as above with w[b,d,k] = sum_r z[b,r] * U[r, d*W+k]; z is (B, R). */
int oracle_lowrank_decode(int64_t B, int64_t D, int32_t W, int32_t R, const double *x, const double *z,
                          const double *U, double *state, int32_t residual, double *y)
{
    if (B < 1 || D < 1 || W < 1 || R < 1) return -2;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            double acc = residual ? x[b * D + d] : 0.0;
            for (int32_t k = 0; k < W; ++k) {
                double wk = 0.0;
                for (int32_t r = 0; r < R; ++r) wk += z[b * R + r] * U[(int64_t)r * D * W + d * W + k];
                double xv = k == 0 ? x[b * D + d] : state[(b * (W - 1) + (k - 1)) * D + d];
                acc += wk * xv;
            }
            y[b * D + d] = acc;
        }
        for (int32_t i = W - 2; i >= 1; --i)
            for (int64_t d = 0; d < D; ++d)
                state[(b * (W - 1) + i) * D + d] = state[(b * (W - 1) + i - 1) * D + d];
        if (W > 1)
            for (int64_t d = 0; d < D; ++d) state[(b * (W - 1)) * D + d] = x[b * D + d];
    }
    return 0;
}

/* State after a prefill of packed sequences: for sequence s = [cu[s], cu[s+1])
 * of the flattened x (B*T, D) (rows of T tokens without cu_seqlens),
 *   state[s, i, d] = x[cu[s+1]-1-i, d] if cu[s+1]-1-i >= cu[s], else 0.
 * state is (n_seqs or B, W-1, D).                                           */
int oracle_state_from_prefill(int64_t B, int64_t T, int64_t D, int32_t W, const double *x,
                              const int32_t *cu_seqlens, int32_t n_seqs, double *state)
{
    if (check_common(B, T, D, W, cu_seqlens, n_seqs, 0, 0)) return -2;
    const int64_t S = (cu_seqlens && n_seqs > 0) ? n_seqs : B;
    for (int64_t sq = 0; sq < S; ++sq) {
        const int64_t lo = (cu_seqlens && n_seqs > 0) ? cu_seqlens[sq] : sq * T;
        const int64_t hi = (cu_seqlens && n_seqs > 0) ? cu_seqlens[sq + 1] : (sq + 1) * T;
        for (int32_t i = 0; i < W - 1; ++i) {
            const int64_t t = hi - 1 - i;
            for (int64_t d = 0; d < D; ++d) state[(sq * (W - 1) + i) * D + d] = t >= lo ? x[t * D + d] : 0.0;
        }
    }
    return 0;
}

/* ------------------------------------------------------- rotary positions */
/*
 * The placement in the pages applies the layer (with its residual) to the
 * query, key and value projections before the rotary position embedding
 * (Methodology, placement).  The rotation itself is not defined there; it is
 * taken from "RoFormer: Enhanced Transformer with Rotary Position Embedding"
 * (Su et al.), Section 3.4.2, general form: a head vector of even dimension
 * hd is split into hd/2 pairs of neighbouring channels (2i, 2i+1), and at
 * position m pair i turns by the angle m * theta_i, theta_i = base^(-2i/hd).
 * Readings: the rotated channels are the first `rot` channels of a row
 * (query heads then key heads, hd channels each; rot a multiple of hd); the
 * remaining channels (values) pass unchanged; the position m of a token is
 * its index inside its own sequence (0 at each sequence start).
 */

/* table[(m*(hd/2) + i)*2 + 0] = cos(m * theta_i), table[... + 1] = sin(m * theta_i)
 * for positions m < max_pos. */
int oracle_rope_table(int64_t max_pos, int32_t hd, double base, double *table)
{
    if (max_pos < 0 || hd < 2 || hd % 2 || !(base > 0.0)) return -2;
    for (int64_t m = 0; m < max_pos; ++m)
        for (int32_t i = 0; i < hd / 2; ++i) {
            const double ang = (double)m * pow(base, -2.0 * i / hd);
            table[(m * (hd / 2) + i) * 2 + 0] = cos(ang);
            table[(m * (hd / 2) + i) * 2 + 1] = sin(ang);
        }
    return 0;
}

/* One row a of D channels turned into b at position m: channels [0, rot)
 * in heads of hd, pair i of each head by the angle sign * m * theta_i; the
 * other channels copied. */
static void rotate_row(int64_t D, int64_t rot, int32_t hd, double base, double m, double sign,
                       const double *a, double *b)
{
    for (int64_t d = rot; d < D; ++d) b[d] = a[d];
    for (int64_t h = 0; h < rot; h += hd)
        for (int32_t i = 0; i < hd / 2; ++i) {
            const double ang = sign * m * pow(base, -2.0 * i / hd);
            const double c = cos(ang), s = sin(ang);
            const double p = a[h + 2 * i], q = a[h + 2 * i + 1];
            b[h + 2 * i] = p * c - q * s;
            b[h + 2 * i + 1] = q * c + p * s;
        }
}

/* Rows [n_lo, n_hi) of v (stored compactly, row n at n - n_lo) rotated into
 * out.  inverse != 0 turns every pair by the opposite angle: the transpose of
 * the rotation, which is what the chain rule applies to an output gradient. */
int oracle_rope(int64_t B, int64_t T, int64_t D, int64_t rot, int32_t hd, double base,
                const int32_t *cu_seqlens, int32_t n_seqs, int32_t inverse,
                int64_t n_lo, int64_t n_hi, const double *v, double *out)
{
    if (check_common(B, T, D, 1, cu_seqlens, n_seqs, n_lo, n_hi)) return -2;
    if (hd < 2 || hd % 2 || rot < 0 || rot > D || rot % hd || !(base > 0.0)) return -2;
    int64_t *seg = segment_starts(B, T, cu_seqlens, n_seqs);
    if (!seg) return -1;
    const double sign = inverse ? -1.0 : 1.0;
#pragma omp parallel for schedule(static)
    for (int64_t n = n_lo; n < n_hi; ++n) {
        const double m = (double)(n - seg[n]);
        rotate_row(D, rot, hd, base, m, sign, v + (n - n_lo) * D, out + (n - n_lo) * D);
    }
    free(seg);
    return 0;
}

/* Decoding: row b of v (B, D) is the newest token of sequence b, at position
 * pos[b] inside it; the row is rotated at that position into out. */
int oracle_rope_at(int64_t B, int64_t D, int64_t rot, int32_t hd, double base, const int32_t *pos,
                   const double *v, double *out)
{
    if (B < 0 || D < 1 || hd < 2 || hd % 2 || rot < 0 || rot > D || rot % hd || !(base > 0.0)) return -2;
    for (int64_t b = 0; b < B; ++b)
        if (pos[b] < 0) return -2;
    for (int64_t b = 0; b < B; ++b)
        rotate_row(D, rot, hd, base, (double)pos[b], 1.0, v + b * D, out + b * D);
    return 0;
}
