/*
 * pdssm_oracle.c -- plain fp64 reference for the Flash PD-SSM forward scan.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this; the library and its kernels never
 * do, and the two share no code.  It is deliberately slow and sequential: one
 * time step after another, exactly as the recurrence is defined, in double
 * precision (complex128 when the state is complex).
 *
 * What is computed (source: "Flash PD-SSM: Memory-Optimized Structured Sparse
 * State-Space Models", gist.science explainer, Technical Summary):
 *
 *   - Methodology, "1. Novel Selection Mechanism (Hard Selection)": a
 *     dictionary of K sparse matrices is fixed in advance; at every step the
 *     K scores pick one matrix by argmax, and that matrix is used as is.  The
 *     selected matrix is a one-hot column selector: column j of P holds a
 *     single 1, in row pi[j].  We store P as the index map pi.
 *   - Methodology, "3. Hardware-Aware Implementation", Phase A: the
 *     recurrence within a chunk is an ordinary sequential recurrence; this
 *     file runs it over the whole sequence.
 *   - The transition is A_t = P_t D_t with D_t diagonal, so
 *         x_t = P_t (d_t * x_{t-1}) + b_t,   y_t = Re( sum_i c_t[i] x_t[i] ).
 *     The pages name the structure (P times D) but print no formula; this
 *     form, the readout without conjugation, and the lowest-index tie-break
 *     of the argmax are the readings this build takes.
 *
 * Inputs are read as the exact double value of the stored bits (fp32, bf16,
 * int16, int32).  Outputs are double.  Index ranges are asserted: a
 * selection outside [0,K) or a map entry outside [0,N) returns an error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage kinds of the selection input. */
enum { ORC_SEL_I32 = 0, ORC_SEL_I16 = 1, ORC_LOGITS_F32 = 2, ORC_LOGITS_BF16 = 3 };

/* Error codes. */
enum { ORC_OK = 0, ORC_BAD_SEL = -1, ORC_BAD_MAP = -2, ORC_BAD_ARG = -3 };

/* bf16 is the upper half of an fp32 bit pattern. */
static double bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Element i of an fp32 or bf16 array, as an exact double. */
static double load_value(const void *base, int64_t i, int is_bf16)
{
    if (is_bf16)
        return bf16_value(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

/*
 * The argmax rule of every hard selection: scanning candidates in order, a
 * later value v replaces the best so far when it is strictly larger, so ties
 * go to the lowest index (the first maximum) and -0 equals +0 under ordinary
 * comparison; a NaN counts as larger than every number, and the first NaN
 * wins.
 */
static int beats(double v, double best_v)
{
    if (isnan(best_v))
        return 0;
    if (isnan(v))
        return 1;
    return v > best_v;
}

/*
 * Hard selection for one step: index mode reads the stored index; logits
 * mode takes the argmax over the K scores.
 */
static int64_t select_step(const void *src, int sel_kind, int64_t step, int32_t K)
{
    if (sel_kind == ORC_SEL_I32)
        return ((const int32_t *)src)[step];
    if (sel_kind == ORC_SEL_I16)
        return ((const int16_t *)src)[step];
    int is_bf16 = (sel_kind == ORC_LOGITS_BF16);
    int64_t row = step * (int64_t)K;
    int64_t best = 0;
    double best_v = load_value(src, row, is_bf16);
    for (int32_t k = 1; k < K; ++k) {
        double v = load_value(src, row + k, is_bf16);
        if (beats(v, best_v)) {
            best = k;
            best_v = v;
        }
    }
    return best;
}

static void set_error(volatile int *err, int code)
{
    if (*err == ORC_OK)
        *err = code;
}

/* sel_out[B,H,L] = the selected dictionary entry of every step. */
int pdssm_oracle_select(const void *src, int sel_kind, int64_t B, int64_t H, int64_t L, int32_t K,
                        int32_t *sel_out)
{
    if (!src || !sel_out || B < 0 || H < 0 || L < 0 || K < 1 || sel_kind < 0 || sel_kind > 3)
        return ORC_BAD_ARG;
    int64_t steps = B * H * L;
    for (int64_t s = 0; s < steps; ++s) {
        int64_t k = select_step(src, sel_kind, s, K);
        if (k < 0 || k >= K)
            return ORC_BAD_SEL;
        sel_out[s] = (int32_t)k;
    }
    return ORC_OK;
}

/*
 * Dictionary pre-compute.  Methodology, "1. Novel Selection Mechanism (Hard
 * Selection)": the K structured matrices come from K dense N x N matrices by
 * a column-wise hardmax, which leaves one non-zero per column, i.e. a one-hot
 * column selector.  For every entry (h,k) and column j:
 *     dict_out[h,k,j] = the row i with the largest m[h,k,i,j]
 * under the same argmax rule as the selection (first maximum, NaN above all).
 * m is [H,K,N,N] row-major (row i, column j), fp32 or bf16 (is_bf16);
 * dict_out is int32 [H,K,N].
 */
int pdssm_oracle_dict_hardmax(const void *m, int is_bf16, int64_t H, int32_t K, int32_t N,
                              int32_t *dict_out)
{
    if (!m || !dict_out || H < 1 || K < 1 || N < 1)
        return ORC_BAD_ARG;
    for (int64_t e = 0; e < H * K; ++e) {
        const int64_t base = e * N * N;   /* matrix (h,k) */
        for (int32_t col = 0; col < N; ++col) {
            int32_t best = 0;
            double best_v = load_value(m, base + col, is_bf16);
            for (int32_t r = 1; r < N; ++r) {
                double v = load_value(m, base + (int64_t)r * N + col, is_bf16);
                if (beats(v, best_v)) {
                    best = r;
                    best_v = v;
                }
            }
            dict_out[e * N + col] = best;
        }
    }
    return ORC_OK;
}

/*
 * Router selection.  Methodology, "1. Novel Selection Mechanism (Hard
 * Selection)": at every step the input u_t produces the K scores by a linear
 * transformation, and the largest score picks the dictionary entry.  With one
 * K-wide block of weights per head (no bias):
 *     logits[b,h,t,k] = sum_{d = 0..D-1 ascending} u[b,t,d] * w[h,k,d]
 *     sel[b,h,t]      = argmax_k logits[b,h,t,k]   (the selection's rule)
 * u is bf16 [B,L,D], w is bf16 [H,K,D]; products of bf16 values are exact in
 * double and the sums are double.  sel_out is int32 [B,H,L]; logits_out, when
 * not NULL, receives the double scores [B,H,L,K].  Rows (b,t) are
 * independent; nthreads > 0 runs that many at once.
 */
int pdssm_oracle_router_select(const uint16_t *u, const uint16_t *w, int64_t B, int64_t L, int64_t H,
                               int32_t K, int32_t D, int32_t *sel_out, double *logits_out,
                               int nthreads)
{
    if (!u || !w || !sel_out || B < 1 || L < 1 || H < 1 || K < 1 || D < 1)
        return ORC_BAD_ARG;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16) if (nthreads > 1)
#endif
    for (int64_t row = 0; row < B * L; ++row) {
        const int64_t bi = row / L, t = row % L;
        const uint16_t *ur = u + row * D;
        for (int64_t h = 0; h < H; ++h) {
            int32_t best = 0;
            double best_v = 0.0;
            for (int32_t k = 0; k < K; ++k) {
                const uint16_t *wr = w + (h * K + k) * (int64_t)D;
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d)
                    acc += bf16_value(ur[d]) * bf16_value(wr[d]);
                if (logits_out)
                    logits_out[((bi * H + h) * L + t) * K + k] = acc;
                if (k == 0 || beats(acc, best_v)) {
                    best = k;
                    best_v = acc;
                }
            }
            sel_out[(bi * H + h) * L + t] = best;
        }
    }
    return ORC_OK;
}

/*
 * The forward scan.  For every sequence (b,h), starting from x0[b,h] (zero
 * when x0 is NULL), for t = 0..L-1:
 *     k   = selected entry of step t
 *     pi  = dict_idx[h,k,:]
 *     x'  = 0;  for j = 0..N-1 (ascending):  x'[pi[j]] += diag[t,j] * x[j]
 *     x'  += b[t,:];  x = x'
 *     y[t] = Re( sum_{i ascending} c[t,i] * x[i] )
 * and x_final[b,h] = x after the last step.
 *
 * Layouts: diag, b, c are [B,H,L,N] (real) or [B,H,L,N,2] (complex,
 * interleaved re/im); diag, x0 are fp32, b and c are fp32 or bf16
 * (bc_bf16).  y_out is double [B,H,L]; xfinal_out (nullable) is double
 * [B,H,N] or [B,H,N,2].  Sequences are independent; nthreads > 0 runs that
 * many of them at once (arithmetic unchanged).
 */
int pdssm_oracle_scan(const void *src, int sel_kind, const int32_t *dict_idx, const float *diag,
                      const void *b, const void *c, const float *x0, int is_complex, int bc_bf16,
                      int64_t B, int64_t H, int64_t L, int32_t N, int32_t K, double *y_out,
                      double *xfinal_out, int nthreads)
{
    if (!src || !dict_idx || !diag || !b || !c || !y_out || B < 0 || H < 0 || L < 0 || N < 1 ||
        K < 1 || sel_kind < 0 || sel_kind > 3)
        return ORC_BAD_ARG;
    const int ncomp = is_complex ? 2 : 1;
    const int64_t BH = B * H;
    volatile int err = ORC_OK;
    (void)nthreads;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t s = 0; s < BH; ++s) {
        const int64_t h = s % H;
        double *x = (double *)calloc((size_t)N * 2, sizeof(double));   /* re, im */
        double *xn = (double *)calloc((size_t)N * 2, sizeof(double));
        if (!x || !xn) {
            set_error(&err, ORC_BAD_ARG);
            free(x);
            free(xn);
            continue;
        }
        if (x0) {
            for (int32_t i = 0; i < N; ++i) {
                x[2 * i] = x0[(s * N + i) * ncomp];
                x[2 * i + 1] = is_complex ? x0[(s * N + i) * ncomp + 1] : 0.0;
            }
        }
        for (int64_t t = 0; t < L && err == ORC_OK; ++t) {
            const int64_t step = s * L + t;
            const int64_t k = select_step(src, sel_kind, step, K);
            if (k < 0 || k >= K) {
                set_error(&err, ORC_BAD_SEL);
                break;
            }
            const int32_t *pi = dict_idx + (h * K + k) * N;
            const int64_t row = step * N;   /* first element of step t */

            for (int32_t i = 0; i < 2 * N; ++i)
                xn[i] = 0.0;
            for (int32_t j = 0; j < N; ++j) {
                const int32_t i = pi[j];
                if (i < 0 || i >= N) {
                    set_error(&err, ORC_BAD_MAP);
                    break;
                }
                const double dr = diag[(row + j) * ncomp];
                const double di = is_complex ? diag[(row + j) * ncomp + 1] : 0.0;
                const double xr = x[2 * j], xi = x[2 * j + 1];
                xn[2 * i] += dr * xr - di * xi;
                xn[2 * i + 1] += dr * xi + di * xr;
            }
            for (int32_t i = 0; i < N; ++i) {
                xn[2 * i] += load_value(b, (row + i) * ncomp, bc_bf16);
                if (is_complex)
                    xn[2 * i + 1] += load_value(b, (row + i) * ncomp + 1, bc_bf16);
            }
            double *tmp = x;
            x = xn;
            xn = tmp;

            double acc = 0.0;
            for (int32_t i = 0; i < N; ++i) {
                const double cr = load_value(c, (row + i) * ncomp, bc_bf16);
                const double ci = is_complex ? load_value(c, (row + i) * ncomp + 1, bc_bf16) : 0.0;
                acc += cr * x[2 * i] - ci * x[2 * i + 1];
            }
            y_out[step] = acc;
        }
        if (xfinal_out) {
            for (int32_t i = 0; i < N; ++i) {
                xfinal_out[(s * N + i) * ncomp] = x[2 * i];
                if (is_complex)
                    xfinal_out[(s * N + i) * ncomp + 1] = x[2 * i + 1];
            }
        }
        free(x);
        free(xn);
    }
    return err;
}

/*
 * The total transition of every sequence, A_{L-1} ... A_1 A_0, which is again
 * a one-hot column selector times a diagonal (the product of such matrices
 * keeps one non-zero per column).  Written per source column j: follow j
 * through the steps,
 *     d_total[j] = prod_t diag[t, p_t(j)],   pi_total[j] = p_L(j),
 * where p_0(j) = j and p_{t+1}(j) = pi_t[p_t(j)].
 * pi_out is int32 [B,H,N]; d_out is double [B,H,N] or [B,H,N,2].
 */
int pdssm_oracle_compose(const void *src, int sel_kind, const int32_t *dict_idx, const float *diag,
                         int is_complex, int64_t B, int64_t H, int64_t L, int32_t N, int32_t K,
                         int32_t *pi_out, double *d_out)
{
    if (!src || !dict_idx || !diag || !pi_out || !d_out || B < 0 || H < 0 || L < 0 || N < 1 ||
        K < 1 || sel_kind < 0 || sel_kind > 3)
        return ORC_BAD_ARG;
    const int ncomp = is_complex ? 2 : 1;
    const int64_t BH = B * H;
    for (int64_t s = 0; s < BH; ++s) {
        const int64_t h = s % H;
        for (int32_t j = 0; j < N; ++j) {
            int32_t p = j;
            double dr = 1.0, di = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t step = s * L + t;
                const int64_t k = select_step(src, sel_kind, step, K);
                if (k < 0 || k >= K)
                    return ORC_BAD_SEL;
                const int64_t e = (step * N + p) * ncomp;
                const double er = diag[e];
                const double ei = is_complex ? diag[e + 1] : 0.0;
                const double nr = er * dr - ei * di;
                const double ni = er * di + ei * dr;
                dr = nr;
                di = ni;
                p = dict_idx[(h * K + k) * N + p];
                if (p < 0 || p >= N)
                    return ORC_BAD_MAP;
            }
            pi_out[s * N + j] = p;
            d_out[(s * N + j) * ncomp] = dr;
            if (is_complex)
                d_out[(s * N + j) * ncomp + 1] = di;
        }
    }
    return ORC_OK;
}

/*
 * Gradients of the forward scan for a real loss whose gradient with respect
 * to y is gy (and, when given, with respect to x_final is gxf).
 *
 * The selection is the hard argmax of the forward pass and receives no
 * gradient (the pages' straight-through estimator for the scores and the
 * dictionary is not specified); b, c, the diagonals and x0 do.  A complex
 * gradient is dL/dRe z + i dL/dIm z.  With the forward states x_t (x_{-1} =
 * x0) kept for every step, and A_t = P_t D_t, the adjoint runs backwards:
 *
 *     lambda_{L-1} = gy_{L-1} conj(c_{L-1}) + gxf
 *     lambda_t     = gy_t conj(c_t) + A_{t+1}^H lambda_{t+1},
 *                    (A^H l)[j] = conj(d[j]) l[pi[j]]   (a gather: the
 *                    transpose of the one-hot column scatter)
 *     gb_t    = lambda_t
 *     gc_t    = gy_t conj(x_t)
 *     gd_t[j] = conj(x_{t-1}[j]) lambda_t[pi_t[j]]
 *     gx0     = A_0^H lambda_0
 *
 * gy is double [B,H,L]; gxf (nullable) double [B,H,N] or [B,H,N,2].  gb, gc,
 * gd are double [B,H,L,N] or [B,H,L,N,2]; gx0 (nullable) double [B,H,N] or
 * [B,H,N,2].  Other arguments as in pdssm_oracle_scan.
 */
int pdssm_oracle_scan_bwd(const void *src, int sel_kind, const int32_t *dict_idx, const float *diag,
                          const void *b, const void *c, const float *x0, const double *gy,
                          const double *gxf, int is_complex, int bc_bf16, int64_t B, int64_t H,
                          int64_t L, int32_t N, int32_t K, double *gb_out, double *gc_out,
                          double *gd_out, double *gx0_out, int nthreads)
{
    if (!src || !dict_idx || !diag || !b || !c || !gy || !gb_out || !gc_out || !gd_out || B < 0 ||
        H < 0 || L < 0 || N < 1 || K < 1 || sel_kind < 0 || sel_kind > 3)
        return ORC_BAD_ARG;
    const int ncomp = is_complex ? 2 : 1;
    const int64_t BH = B * H;
    volatile int err = ORC_OK;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t s = 0; s < BH; ++s) {
        const int64_t h = s % H;
        /* xs[t+1] = x_t for t = -1..L-1 (re, im), and the step maps. */
        double *xs = (double *)calloc((size_t)(L + 1) * N * 2, sizeof(double));
        int32_t *maps = (int32_t *)malloc((size_t)(L > 0 ? L : 1) * N * sizeof(int32_t));
        double *lam = (double *)calloc((size_t)N * 2, sizeof(double));
        double *lnew = (double *)calloc((size_t)N * 2, sizeof(double));
        if (!xs || !maps || !lam || !lnew) {
            set_error(&err, ORC_BAD_ARG);
            free(xs);
            free(maps);
            free(lam);
            free(lnew);
            continue;
        }
        if (x0 != NULL) {
            for (int32_t i = 0; i < N; ++i) {
                xs[2 * i] = x0[(s * N + i) * ncomp];
                xs[2 * i + 1] = is_complex ? x0[(s * N + i) * ncomp + 1] : 0.0;
            }
        }
        /* Forward: the states, exactly as in pdssm_oracle_scan. */
        for (int64_t t = 0; t < L && err == ORC_OK; ++t) {
            const int64_t step = s * L + t;
            const int64_t k = select_step(src, sel_kind, step, K);
            if (k < 0 || k >= K) {
                set_error(&err, ORC_BAD_SEL);
                break;
            }
            const int32_t *pi = dict_idx + (h * K + k) * N;
            const int64_t row = step * N;
            const double *x = xs + (size_t)t * N * 2;
            double *xn = xs + (size_t)(t + 1) * N * 2;
            for (int32_t j = 0; j < N; ++j) {
                const int32_t i = pi[j];
                if (i < 0 || i >= N) {
                    set_error(&err, ORC_BAD_MAP);
                    break;
                }
                maps[t * N + j] = i;
                const double ar = diag[(row + j) * ncomp];
                const double ai = is_complex ? diag[(row + j) * ncomp + 1] : 0.0;
                xn[2 * i] += ar * x[2 * j] - ai * x[2 * j + 1];
                xn[2 * i + 1] += ar * x[2 * j + 1] + ai * x[2 * j];
            }
            for (int32_t i = 0; i < N; ++i) {
                xn[2 * i] = xn[2 * i] + load_value(b, (row + i) * ncomp, bc_bf16);
                if (is_complex)
                    xn[2 * i + 1] = xn[2 * i + 1] + load_value(b, (row + i) * ncomp + 1, bc_bf16);
            }
        }
        if (err != ORC_OK) {
            free(xs);
            free(maps);
            free(lam);
            free(lnew);
            continue;
        }
        /* Backward. */
        if (gxf) {
            for (int32_t i = 0; i < N; ++i) {
                lam[2 * i] = gxf[(s * N + i) * ncomp];
                lam[2 * i + 1] = is_complex ? gxf[(s * N + i) * ncomp + 1] : 0.0;
            }
        }
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t step = s * L + t;
            const int64_t row = step * N;
            const double g = gy[step];
            /* lambda_t = (carried part) + gy_t conj(c_t) */
            for (int32_t i = 0; i < N; ++i) {
                const double cr = load_value(c, (row + i) * ncomp, bc_bf16);
                const double ci = is_complex ? load_value(c, (row + i) * ncomp + 1, bc_bf16) : 0.0;
                lam[2 * i] += g * cr;
                lam[2 * i + 1] += -g * ci;
            }
            const double *xt = xs + (size_t)(t + 1) * N * 2;   /* x_t */
            const double *xp = xs + (size_t)t * N * 2;         /* x_{t-1} */
            const int32_t *pi = maps + t * N;
            for (int32_t i = 0; i < N; ++i) {
                const int64_t e = (row + i) * ncomp;
                gb_out[e] = lam[2 * i];
                gc_out[e] = g * xt[2 * i];
                if (is_complex) {
                    gb_out[e + 1] = lam[2 * i + 1];
                    gc_out[e + 1] = -g * xt[2 * i + 1];
                }
            }
            /* gd_t[j] = conj(x_{t-1}[j]) lambda_t[pi[j]];
               lambda_{t-1} (before its own readout term) = conj(d_t[j]) lambda_t[pi[j]] */
            for (int32_t j = 0; j < N; ++j) {
                const double lr = lam[2 * pi[j]], li = lam[2 * pi[j] + 1];
                const double xr = xp[2 * j], xi = xp[2 * j + 1];
                const int64_t e = (row + j) * ncomp;
                gd_out[e] = xr * lr + xi * li;
                if (is_complex)
                    gd_out[e + 1] = xr * li - xi * lr;
                const double dr = diag[e];
                const double di = is_complex ? diag[e + 1] : 0.0;
                lnew[2 * j] = dr * lr + di * li;
                lnew[2 * j + 1] = dr * li - di * lr;
            }
            double *tmp = lam;
            lam = lnew;
            lnew = tmp;
        }
        if (gx0_out) {
            for (int32_t i = 0; i < N; ++i) {
                gx0_out[(s * N + i) * ncomp] = lam[2 * i];
                if (is_complex)
                    gx0_out[(s * N + i) * ncomp + 1] = lam[2 * i + 1];
            }
        }
        free(xs);
        free(maps);
        free(lam);
        free(lnew);
    }
    return err;
}
