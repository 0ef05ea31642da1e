/*
 * oracle.c -- plain, slow fp64 CPU reference for the batch-invariant kernels.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code with the HIP library.
 *
 * Every reduction below runs sequentially in ascending index order in fp64.
 * OpenMP is used only across independent rows / (row, head) pairs, never
 * inside a reduction, so results do not depend on the thread count.
 *
 * Sources (pages on LLM inference nondeterminism):
 *   [TML-explainer]  devpress.csdn.net explainer of Thinking Machines' "Defeating
 *                    Nondeterminism in LLM Inference" (sections 3.1 RMSNorm,
 *                    3.2 Matmul, 3.3 Attention).
 *   [BIK-notes]      tom-jerr.github.io "Batch-Invariant Kernel" reading notes
 *                    (sections RMSNorm, GEMM, Flash Attention).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below will use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads the row loops use (for timing the oracle
 * on one core or on all of them; the arithmetic of every row is unchanged). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* bf16 rounding: nearest value with 8 significant bits, ties to even.       */
/* bf16 = 1 sign bit, 8 exponent bits (same range as binary32), 7 stored     */
/* fraction bits.  Written from that definition, not from any bit trick.     */
/* ------------------------------------------------------------------------ */
double oracle_round_bf16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    double f = frexp(x, &e);            /* x = f * 2^e, 0.5 <= |f| < 1 */
    if (e < -125) e = -125;             /* below 2^-126 the spacing stays 2^-133 */
    double spacing_exp = (double)(e - 8);
    double scaled = ldexp(x, -(e - 8));  /* x / spacing, exact */
    double r = nearbyint(scaled);        /* default mode: round half to even */
    double y = ldexp(r, (int)spacing_exp);
    const double bf16_max = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (fabs(y) > bf16_max) return copysign(INFINITY, x);
    return y;
}

void oracle_round_bf16_array(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm  ([BIK-notes] RMSNorm formula; [TML-explainer] 3.1):               */
/*   y[i,j] = x[i,j] * 1/sqrt( (1/d) * sum_j x[i,j]^2 + eps ) * gamma[j]      */
/* eps sits inside the square root, added to the mean over the d features.   */
/* ------------------------------------------------------------------------ */
void oracle_rmsnorm(const double* x, int64_t ldx, const double* gamma,
                    double* y, int64_t ldy, int64_t M, int64_t d, double eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const double* xr = x + i * ldx;
        double ss = 0.0;
        for (int64_t j = 0; j < d; ++j) ss += xr[j] * xr[j];
        double r = 1.0 / sqrt(ss / (double)d + eps);
        double* yr = y + i * ldy;
        for (int64_t j = 0; j < d; ++j) yr[j] = xr[j] * r * gamma[j];
    }
}

/* ------------------------------------------------------------------------ */
/* GEMM  ([TML-explainer] 3.2: C[i,j] = sum_k A[i,k] * B[k,j]):              */
/*   A [M,K] row-major (lda), W [K,N] row-major (ldw), C [M,N] (ldc).        */
/* Each C[i,j] is accumulated over k = 0, 1, ..., K-1 in that order.         */
/* ------------------------------------------------------------------------ */
void oracle_gemm(const double* A, int64_t lda, const double* W, int64_t ldw,
                 double* C, int64_t ldc, int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* cr = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) cr[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[i * lda + k];
            const double* wr = W + k * ldw;
            for (int64_t j = 0; j < N; ++j) cr[j] += a * wr[j];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Causal grouped-query attention for ONE sequence ([TML-explainer] 3.3:     */
/* two reductions over the KV length, first Q K^T then softmax(.) V).        */
/*   q   [nq, Hq, D]   query rows; row i sits at absolute position pos[i]    */
/*   k,v [L, Hkv, D]   the sequence's keys / values in logical token order   */
/*   out [nq, Hq, D]                                                         */
/* Row i attends to keys 0..pos[i] (a query at position p sees the p earlier */
/* tokens and itself).  Query head h reads KV head h / (Hq/Hkv).             */
/* softmax with the row maximum subtracted before exp (exact in reals).      */
/* Returns 0, or -1 if some pos[i] is outside [0, L).                        */
/* ------------------------------------------------------------------------ */
int oracle_attention(const double* q, const int64_t* pos, const double* k,
                     const double* v, int64_t nq, int64_t L, int64_t Hq,
                     int64_t Hkv, int64_t D, double scale, double* out)
{
    for (int64_t i = 0; i < nq; ++i)
        if (pos[i] < 0 || pos[i] >= L) return -1;
    const int64_t group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < nq; ++i) {
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / group;
            const int64_t n = pos[i] + 1;
            const double* qr = q + (i * Hq + h) * D;
            double* s = (double*)malloc((size_t)n * sizeof(double));
            if (!s) { bad = 1; continue; }
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                const double* kr = k + (j * Hkv + g) * D;
                double dot = 0.0;
                for (int64_t t = 0; t < D; ++t) dot += qr[t] * kr[t];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            double z = 0.0;
            for (int64_t j = 0; j < n; ++j) { s[j] = exp(s[j] - m); z += s[j]; }
            double* o = out + (i * Hq + h) * D;
            for (int64_t t = 0; t < D; ++t) o[t] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double w = s[j] / z;
                const double* vr = v + (j * Hkv + g) * D;
                for (int64_t t = 0; t < D; ++t) o[t] += w * vr[t];
            }
            free(s);
        }
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* The same attention evaluated the way the method splits it, in fp64:       */
/*  * fixed-size split-KV ([TML-explainer] 3.3 fixed 256-token split example;*/
/*    [BIK-notes] Flash Attention, fixed-size Split-KV): chunk c holds the   */
/*    keys [c*chunk, (c+1)*chunk) intersected with [0, pos], counted from    */
/*    absolute position 0;                                                   */
/*  * per chunk a partial (m, l, o): m = max score, l = sum exp(s - m),      */
/*    o = sum exp(s - m) v;                                                  */
/*  * the partials merged by a binary tree padded to a fixed depth           */
/*    ([BIK-notes] Flash Attention: merge with a chunk-count-independent     */
/*    binary tree of fixed depth): 2^depth leaves, leaves past the last      */
/*    chunk are the identity (-inf, 0, 0), node = combine(left, right) with  */
/*    m = max(m1,m2), a_i = exp(m_i - m), l = a1 l1 + a2 l2, o = a1 o1 + a2 o2.*/
/*  * out = o / l.                                                           */
/* In exact arithmetic this equals oracle_attention.  Returns 0, -1 on bad   */
/* positions, -3 if a row needs more than 2^depth chunks.                    */
/* ------------------------------------------------------------------------ */
typedef struct { double m, l; double* o; } oracle_partial;

static void combine_into(oracle_partial* left, const oracle_partial* right, int64_t D)
{
    /* identity (-inf, 0, 0) on both sides stays the identity */
    if (left->m == -INFINITY && right->m == -INFINITY) return;
    const double m = left->m > right->m ? left->m : right->m;
    const double a1 = exp(left->m - m);
    const double a2 = exp(right->m - m);
    left->l = a1 * left->l + a2 * right->l;
    for (int64_t t = 0; t < D; ++t) left->o[t] = a1 * left->o[t] + a2 * right->o[t];
    left->m = m;
}

int oracle_attention_chunked(const double* q, const int64_t* pos, const double* k,
                             const double* v, int64_t nq, int64_t L, int64_t Hq,
                             int64_t Hkv, int64_t D, double scale, int64_t chunk,
                             int64_t depth, double* out)
{
    for (int64_t i = 0; i < nq; ++i)
        if (pos[i] < 0 || pos[i] >= L) return -1;
    const int64_t leaves = (int64_t)1 << depth;
    for (int64_t i = 0; i < nq; ++i)
        if ((pos[i] + chunk) / chunk > leaves) return -3;
    const int64_t group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < nq; ++i) {
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / group;
            const int64_t n = pos[i] + 1;               /* keys 0..pos */
            const double* qr = q + (i * Hq + h) * D;
            oracle_partial* node = (oracle_partial*)malloc((size_t)leaves * sizeof(oracle_partial));
            double* obuf = (double*)calloc((size_t)(leaves * D), sizeof(double));
            if (!node || !obuf) { free(node); free(obuf); bad = 1; continue; }
            for (int64_t c = 0; c < leaves; ++c) {
                node[c].m = -INFINITY; node[c].l = 0.0; node[c].o = obuf + c * D;
                const int64_t j0 = c * chunk;
                const int64_t j1 = (j0 + chunk < n) ? j0 + chunk : n;
                if (j0 >= n) continue;                  /* padding leaf */
                double m = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    const double* kr = k + (j * Hkv + g) * D;
                    double dot = 0.0;
                    for (int64_t t = 0; t < D; ++t) dot += qr[t] * kr[t];
                    const double s = scale * dot;
                    if (s > m) m = s;
                }
                double l = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    const double* kr = k + (j * Hkv + g) * D;
                    double dot = 0.0;
                    for (int64_t t = 0; t < D; ++t) dot += qr[t] * kr[t];
                    const double p = exp(scale * dot - m);
                    l += p;
                    const double* vr = v + (j * Hkv + g) * D;
                    for (int64_t t = 0; t < D; ++t) node[c].o[t] += p * vr[t];
                }
                node[c].m = m; node[c].l = l;
            }
            /* fixed-depth tree: level by level, node i <- combine(2i, 2i+1) */
            for (int64_t width = leaves; width > 1; width /= 2) {
                for (int64_t a = 0; a < width / 2; ++a) {
                    oracle_partial left = node[2 * a];
                    combine_into(&left, &node[2 * a + 1], D);
                    /* move the merged node to slot a (its o buffer stays put) */
                    node[a].m = left.m; node[a].l = left.l;
                    if (node[a].o != left.o)
                        for (int64_t t = 0; t < D; ++t) node[a].o[t] = left.o[t];
                }
            }
            double* o = out + (i * Hq + h) * D;
            for (int64_t t = 0; t < D; ++t) o[t] = node[0].o[t] / node[0].l;
            free(obuf); free(node);
        }
    }
    return bad ? -2 : 0;
}

/* Chunk partition of a row at absolute position pos (keys 0..pos):          */
/* writes the number of valid keys of chunk c into counts[c], returns the    */
/* number of chunks.  counts must hold at least (pos + chunk) / chunk entries.*/
int64_t oracle_chunk_partition(int64_t n_keys, int64_t chunk, int64_t* counts)
{
    int64_t c = 0;
    for (int64_t j0 = 0; j0 < n_keys; j0 += chunk, ++c)
        counts[c] = (n_keys - j0 < chunk) ? n_keys - j0 : chunk;
    return c;
}
