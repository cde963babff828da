/*
 * more_oracle.c -- fp64 CPU oracle for the fused low-rank MoE router.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP product path
 * never calls it, shares no code, header, table or helper with it, and
 * fails loudly instead of falling back to it.
 *
 * Source of the method: "MoRE: Scaling mixture of experts with hardware-aware
 * low-rank routing" (Wong, Goel, Boix-Adsera).
 *   - §2 (MoE layer / MoRE layer): the standard router g(x) = softmax(TopK(Rx))
 *     and the low-rank router, which replaces R by a product of a rank-r
 *     down-projection and an up-projection.  In this library's convention the
 *     down-projection R1 is h x r and the up-projection R2 is r x M (both
 *     row-major), so the logits of token x are (x R1) R2; the paper's factors
 *     are the transposes of these.
 *   - App. F, eq. (5): the logits matrix of all tokens and experts.
 *   - App. F.1, Algorithm 1 and Fig. 12: the inference kernel returns the
 *     exact top-k values and indices; the gate weights are a softmax over the
 *     k selected logits.
 *   - App. F.2.1, eq. (6): the full softmax P = exp(l) / Z over all M experts,
 *     used for the FULL_SOFTMAX gate (P evaluated at the selected experts, not
 *     renormalised) and for the log-sum-exp output.
 *
 * What the oracle computes, per token n, in fp64 on the exact values of the
 * stored inputs (bf16 bits or fp32; fp64 accepted for tests):
 *   1. z = x_n R1                       (r values; skipped for full rank)
 *   2. l = z R2 + b   (or l = x_n W + b for the full-rank router; b = 0 if absent)
 *   3. order all M experts by (l descending, index ascending) with qsort and
 *      keep the first k: ties go to the lower expert index.
 *   4. TOPK_SOFTMAX: g_j = exp(l_j - l_(1)) / sum_{i in S} exp(l_i - l_(1)).
 *      FULL_SOFTMAX: m = max l, Z = sum over all M of exp(l - m),
 *      lse = m + log Z, g_j = exp(l_j - lse).
 *   5. side outputs: the k selected logits, l_(k), l_(k+1) (-inf if k = M)
 *      and max_j |l_j|, the data of the gap rule used to compare against.
 * Balancing statistics (App. F.2.1, eq. (7)): psum_i = sum over tokens of the
 * full-softmax probability P_{n,i} = exp(l_{n,i} - m_n) / Z_n of eq. (6),
 * with m_n and Z_n taken over all M experts of the biased logits.
 * Backward (App. F.2.2, eq. (10)-(12), Algorithm 3), per token n with the
 * selection idx held fixed: g_n = sum_i pbar_i P_{n,i};
 * ybar_{n,j} = P_{n,j} (pbar_j - g_n) + sum of tvbar_{n,c} over the slots c
 * with idx_{n,c} = j; zbar = ybar R2^T; xbar = zbar R1^T; summed over tokens:
 * R2bar += z^T ybar, R1bar += x^T zbar, bbar += ybar.
 * No blocking, fusion or reordering beyond these definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_DT_BF16 = 0, OR_DT_F32 = 1, OR_DT_F64 = 2 };
enum { OR_GATE_TOPK = 0, OR_GATE_FULL = 1 };
enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_NONFINITE = 2, OR_ERR_NOMEM = 3 };

static double load_elem(int dt, const void* p, int64_t i) {
    if (dt == OR_DT_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dt == OR_DT_F32) return (double)((const float*)p)[i];
    return ((const double*)p)[i];
}

static int all_finite(int dt, const void* p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(load_elem(dt, p, i))) return 0;
    return 1;
}

typedef struct { double v; int64_t idx; } entry_t;

/* (value descending, index ascending): a total order, so qsort's result is unique. */
static int cmp_entry(const void* a, const void* b) {
    const entry_t* x = (const entry_t*)a;
    const entry_t* y = (const entry_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/* Logits of one token into l[0..M). */
static void token_logits(int dt, const void* X, int64_t n, int64_t h, const void* A, int64_t r,
                         const void* B, int64_t M, const float* bias, int fullrank,
                         double* x, double* z, double* l) {
    for (int64_t i = 0; i < h; ++i) x[i] = load_elem(dt, X, n * h + i);
    if (fullrank) {
        /* l_m = sum_i x_i W[i][m] + b_m, W is h x M */
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0;
            for (int64_t i = 0; i < h; ++i) s += x[i] * load_elem(dt, A, i * M + m);
            l[m] = s + (bias ? (double)bias[m] : 0.0);
        }
        return;
    }
    /* z_j = sum_i x_i R1[i][j], R1 is h x r */
    for (int64_t j = 0; j < r; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < h; ++i) s += x[i] * load_elem(dt, A, i * r + j);
        z[j] = s;
    }
    /* l_m = sum_j z_j R2[j][m] + b_m, R2 is r x M */
    for (int64_t m = 0; m < M; ++m) {
        double s = 0.0;
        for (int64_t j = 0; j < r; ++j) s += z[j] * load_elem(dt, B, j * M + m);
        l[m] = s + (bias ? (double)bias[m] : 0.0);
    }
}

static int route_impl(int dt, const void* X, int64_t N, int64_t h, const void* A, int64_t r,
                      const void* B, int64_t M, const float* bias, int k, int gate, int fullrank,
                      int32_t* idx_out, double* gate_out, double* logit_out, double* lse_out,
                      double* kth_out, double* kp1_out, double* maxabs_out, int nthreads) {
    if (dt < OR_DT_BF16 || dt > OR_DT_F64) return OR_ERR_ARG;
    if (gate != OR_GATE_TOPK && gate != OR_GATE_FULL) return OR_ERR_ARG;
    if (!X || !A || (!fullrank && !B) || !idx_out || !gate_out) return OR_ERR_ARG;
    if (N < 0 || h < 1 || M < 1 || (!fullrank && r < 1) || k < 1 || k > M) return OR_ERR_ARG;
    if (!all_finite(dt, X, N * h)) return OR_ERR_NONFINITE;
    if (fullrank) {
        if (!all_finite(dt, A, h * M)) return OR_ERR_NONFINITE;
    } else {
        if (!all_finite(dt, A, h * r) || !all_finite(dt, B, r * M)) return OR_ERR_NONFINITE;
    }
    if (bias && !all_finite(OR_DT_F32, bias, M)) return OR_ERR_NONFINITE;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    const int T = omp_get_max_threads();
#else
    (void)nthreads;
    const int T = 1;
#endif
    /* Per-thread scratch, allocated up front so every thread enters the loop. */
    double* xs = (double*)malloc(sizeof(double) * (size_t)h * (size_t)T);
    double* zs = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1) * (size_t)T);
    double* ls = (double*)malloc(sizeof(double) * (size_t)M * (size_t)T);
    entry_t* es = (entry_t*)malloc(sizeof(entry_t) * (size_t)M * (size_t)T);
    if (!xs || !zs || !ls || !es) {
        free(xs);
        free(zs);
        free(ls);
        free(es);
        return OR_ERR_NOMEM;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
#ifdef _OPENMP
        const int t = omp_get_thread_num();
#else
        const int t = 0;
#endif
        double* x = xs + (size_t)t * (size_t)h;
        double* z = zs + (size_t)t * (size_t)(r > 0 ? r : 1);
        double* l = ls + (size_t)t * (size_t)M;
        entry_t* e = es + (size_t)t * (size_t)M;
        token_logits(dt, X, n, h, A, r, B, M, bias, fullrank, x, z, l);
        double maxabs = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            e[m].v = l[m];
            e[m].idx = m;
            if (fabs(l[m]) > maxabs) maxabs = fabs(l[m]);
        }
        qsort(e, (size_t)M, sizeof(entry_t), cmp_entry);
        const double top = e[0].v;
        double lse = 0.0;
        if (gate == OR_GATE_FULL) {
            double Z = 0.0;
            for (int64_t m = 0; m < M; ++m) Z += exp(l[m] - top);
            lse = top + log(Z);
        }
        double denom = 0.0;
        for (int j = 0; j < k; ++j) denom += exp(e[j].v - top);
        for (int j = 0; j < k; ++j) {
            idx_out[n * k + j] = (int32_t)e[j].idx;
            gate_out[n * k + j] = (gate == OR_GATE_FULL) ? exp(e[j].v - lse)
                                                          : exp(e[j].v - top) / denom;
            if (logit_out) logit_out[n * k + j] = e[j].v;
        }
        if (lse_out) lse_out[n] = (gate == OR_GATE_FULL) ? lse : NAN;
        if (kth_out) kth_out[n] = e[k - 1].v;
        if (kp1_out) kp1_out[n] = (k < M) ? e[k].v : -INFINITY;
        if (maxabs_out) maxabs_out[n] = maxabs;
    }
    free(xs);
    free(zs);
    free(ls);
    free(es);
    return OR_OK;
}

int oracle_route_lowrank(int dt, const void* X, int64_t N, int64_t h, const void* R1, int64_t r,
                         const void* R2, int64_t M, const float* bias, int k, int gate,
                         int32_t* idx_out, double* gate_out, double* logit_out, double* lse_out,
                         double* kth_out, double* kp1_out, double* maxabs_out, int nthreads) {
    return route_impl(dt, X, N, h, R1, r, R2, M, bias, k, gate, 0, idx_out, gate_out, logit_out,
                      lse_out, kth_out, kp1_out, maxabs_out, nthreads);
}

int oracle_route_fullrank(int dt, const void* X, int64_t N, int64_t h, const void* W, int64_t M,
                          const float* bias, int k, int gate, int32_t* idx_out, double* gate_out,
                          double* logit_out, double* lse_out, double* kth_out, double* kp1_out,
                          double* maxabs_out, int nthreads) {
    return route_impl(dt, X, N, h, W, 0, NULL, M, bias, k, gate, 1, idx_out, gate_out, logit_out,
                      lse_out, kth_out, kp1_out, maxabs_out, nthreads);
}

/* All N x M logits (small inputs only: tests use it for the invariants). */
int oracle_logits(int dt, const void* X, int64_t N, int64_t h, const void* A, int64_t r,
                  const void* B, int64_t M, const float* bias, int fullrank, double* out) {
    if (dt < OR_DT_BF16 || dt > OR_DT_F64 || !X || !A || (!fullrank && !B) || !out) return OR_ERR_ARG;
    if (N < 0 || h < 1 || M < 1 || (!fullrank && r < 1)) return OR_ERR_ARG;
    double* x = (double*)malloc(sizeof(double) * (size_t)h);
    double* z = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
    if (!x || !z) {
        free(x);
        free(z);
        return OR_ERR_NOMEM;
    }
    for (int64_t n = 0; n < N; ++n) token_logits(dt, X, n, h, A, r, B, M, bias, fullrank, x, z, out + n * M);
    free(x);
    free(z);
    return OR_OK;
}

/*
 * Logits of chosen experts: out[n * k + j] = l_{n, idx[n k + j]}, the same
 * definition as oracle_logits (z = x R1, l = z R2 + b, or l = x W + b for
 * full rank) evaluated only at the k given experts of each token, so that a
 * selection made elsewhere can be checked against the fp64 logits of the
 * experts it names.  An index outside [0, M) gives NaN.
 */
int oracle_logits_at(int dt, const void* X, int64_t N, int64_t h, const void* A, int64_t r,
                     const void* B, int64_t M, const float* bias, int fullrank, int k,
                     const int32_t* idx, double* out, int nthreads) {
    if (dt < OR_DT_BF16 || dt > OR_DT_F64 || !X || !A || (!fullrank && !B) || !idx || !out) return OR_ERR_ARG;
    if (N < 0 || h < 1 || M < 1 || (!fullrank && r < 1) || k < 1) return OR_ERR_ARG;
    int T = 1;
#ifdef _OPENMP
    T = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    (void)nthreads;
    const size_t zr = (size_t)(r > 0 ? r : 1);
    double* zs = (double*)malloc(sizeof(double) * (size_t)T * zr);
    if (!zs) return OR_ERR_NOMEM;
#ifdef _OPENMP
#pragma omp parallel for num_threads(T) schedule(static)
#endif
    for (int64_t n = 0; n < N; ++n) {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
        double* z = zs + (size_t)t * zr;
        if (!fullrank) {
            /* z_j = sum_i x_i R1[i][j] */
            for (int64_t j = 0; j < r; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < h; ++i) s += load_elem(dt, X, n * h + i) * load_elem(dt, A, i * r + j);
                z[j] = s;
            }
        }
        for (int c = 0; c < k; ++c) {
            const int64_t m = idx[n * k + c];
            if (m < 0 || m >= M) {
                out[n * k + c] = NAN;
                continue;
            }
            double s = 0.0;
            if (fullrank) {
                for (int64_t i = 0; i < h; ++i) s += load_elem(dt, X, n * h + i) * load_elem(dt, A, i * M + m);
            } else {
                for (int64_t j = 0; j < r; ++j) s += z[j] * load_elem(dt, B, j * M + m);
            }
            out[n * k + c] = s + (bias ? (double)bias[m] : 0.0);
        }
    }
    free(zs);
    return OR_OK;
}

/*
 * Column sums of the row-wise full softmax (eq. (6), (7)): psum[i] = sum_n
 * P_{n,i}.  Per token: logits as above, m = max l, Z = sum exp(l - m),
 * P = exp(l - m) / Z; each thread sums its tokens, the thread sums are added
 * at the end.
 */
int oracle_softmax_colsum(int dt, const void* X, int64_t N, int64_t h, const void* A, int64_t r,
                          const void* B, int64_t M, const float* bias, int fullrank, double* psum_out,
                          int nthreads) {
    if (dt < OR_DT_BF16 || dt > OR_DT_F64 || !X || !A || (!fullrank && !B) || !psum_out) return OR_ERR_ARG;
    if (N < 0 || h < 1 || M < 1 || (!fullrank && r < 1)) return OR_ERR_ARG;
    if (!all_finite(dt, X, N * h) || !all_finite(dt, A, fullrank ? h * M : h * r) ||
        (!fullrank && !all_finite(dt, B, r * M)) || (bias && !all_finite(OR_DT_F32, bias, M)))
        return OR_ERR_NONFINITE;
    int T = 1;
#ifdef _OPENMP
    T = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    (void)nthreads;
    const size_t zr = (size_t)(r > 0 ? r : 1);
    double* part = (double*)calloc((size_t)T * (size_t)M, sizeof(double));
    double* xs = (double*)malloc(sizeof(double) * (size_t)T * (size_t)h);
    double* zs = (double*)malloc(sizeof(double) * (size_t)T * zr);
    double* ls = (double*)malloc(sizeof(double) * (size_t)T * (size_t)M);
    if (!part || !xs || !zs || !ls) {
        free(part);
        free(xs);
        free(zs);
        free(ls);
        return OR_ERR_NOMEM;
    }
#ifdef _OPENMP
#pragma omp parallel for num_threads(T) schedule(static)
#endif
    for (int64_t n = 0; n < N; ++n) {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
        double* l = ls + (size_t)t * (size_t)M;
        double* acc = part + (size_t)t * (size_t)M;
        token_logits(dt, X, n, h, A, r, B, M, bias, fullrank, xs + (size_t)t * (size_t)h, zs + (size_t)t * zr, l);
        double m = l[0];
        for (int64_t i = 1; i < M; ++i) m = l[i] > m ? l[i] : m;
        double Z = 0.0;
        for (int64_t i = 0; i < M; ++i) Z += exp(l[i] - m);
        for (int64_t i = 0; i < M; ++i) acc[i] += exp(l[i] - m) / Z;
    }
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0;
        for (int t = 0; t < T; ++t) s += part[(size_t)t * (size_t)M + (size_t)i];
        psum_out[i] = s;
    }
    free(part);
    free(xs);
    free(zs);
    free(ls);
    return OR_OK;
}

/*
 * Gradients of F = sum_{n,c} tvbar_{n,c} l_{n, idx_{n,c}} + sum_i pbar_i psum_i
 * (the prediction loss through the selected logits and the balancing loss
 * through psum, eq. (9)-(12)) with respect to X, R1, R2 and the bias, the
 * selection idx held fixed.  pbar may be NULL (zero).  Outputs (fp64):
 * xbar N x h, r1bar h x r, r2bar r x M, bbar M.
 */
int oracle_backward_lowrank(int dt, const void* X, int64_t N, int64_t h, const void* R1, int64_t r,
                            const void* R2, int64_t M, const float* bias, int k, const int32_t* idx,
                            const double* tvbar, const double* pbar, double* xbar, double* r1bar,
                            double* r2bar, double* bbar, int nthreads) {
    if (dt < OR_DT_BF16 || dt > OR_DT_F64 || !X || !R1 || !R2 || !idx || !tvbar || !xbar || !r1bar || !r2bar ||
        !bbar)
        return OR_ERR_ARG;
    if (N < 0 || h < 1 || M < 1 || r < 1 || k < 1 || k > M) return OR_ERR_ARG;
    for (int64_t i = 0; i < N * k; ++i)
        if (idx[i] < 0 || idx[i] >= M) return OR_ERR_ARG;
    int T = 1;
#ifdef _OPENMP
    T = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    (void)nthreads;
    const size_t per = (size_t)(h * r + r * M + M);
    double* part = (double*)calloc((size_t)T * per, sizeof(double));
    double* work = (double*)malloc(sizeof(double) * (size_t)T * (size_t)(h + 2 * r + 2 * M));
    if (!part || !work) {
        free(part);
        free(work);
        return OR_ERR_NOMEM;
    }
#ifdef _OPENMP
#pragma omp parallel for num_threads(T) schedule(static)
#endif
    for (int64_t n = 0; n < N; ++n) {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
        double* x = work + (size_t)t * (size_t)(h + 2 * r + 2 * M);
        double* z = x + h;
        double* zb = z + r;
        double* l = zb + r;
        double* yb = l + M;
        double* r1b = part + (size_t)t * per;
        double* r2b = r1b + h * r;
        double* bb = r2b + r * M;
        token_logits(dt, X, n, h, R1, r, R2, M, bias, 0, x, z, l);
        double m = l[0];
        for (int64_t i = 1; i < M; ++i) m = l[i] > m ? l[i] : m;
        double Z = 0.0;
        for (int64_t i = 0; i < M; ++i) Z += exp(l[i] - m);
        double g = 0.0;
        for (int64_t i = 0; i < M; ++i) {
            yb[i] = exp(l[i] - m) / Z;   /* P_{n,i} for now */
            g += (pbar ? pbar[i] : 0.0) * yb[i];
        }
        for (int64_t i = 0; i < M; ++i) yb[i] = yb[i] * ((pbar ? pbar[i] : 0.0) - g);
        for (int c = 0; c < k; ++c) yb[idx[n * k + c]] += tvbar[n * k + c];
        for (int64_t j = 0; j < r; ++j) {
            double s = 0.0;
            for (int64_t i = 0; i < M; ++i) s += yb[i] * load_elem(dt, R2, j * M + i);
            zb[j] = s;
        }
        for (int64_t i = 0; i < h; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < r; ++j) s += zb[j] * load_elem(dt, R1, i * r + j);
            xbar[n * h + i] = s;
        }
        for (int64_t i = 0; i < h; ++i)
            for (int64_t j = 0; j < r; ++j) r1b[i * r + j] += x[i] * zb[j];
        for (int64_t j = 0; j < r; ++j)
            for (int64_t i = 0; i < M; ++i) r2b[j * M + i] += z[j] * yb[i];
        for (int64_t i = 0; i < M; ++i) bb[i] += yb[i];
    }
    for (size_t q = 0; q < per; ++q) {
        double s = 0.0;
        for (int t = 0; t < T; ++t) s += part[(size_t)t * per + q];
        if (q < (size_t)(h * r)) r1bar[q] = s;
        else if (q < (size_t)(h * r + r * M)) r2bar[q - (size_t)(h * r)] = s;
        else bbar[q - (size_t)(h * r + r * M)] = s;
    }
    free(part);
    free(work);
    return OR_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
