/*
 * fp64 CPU oracle for the FlowCache per-step hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * reference that the GPU kernels are checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, constant or helper with the HIP library.
 *
 * Source of every formula: the page "Flow Caching for Autoregressive Video
 * Generation" (papernotes.org ICLR 2026 digest), section 方法详解 / 关键设计
 * ("Key designs"), item 3 "joint importance-redundancy KV cache compression":
 *   - importance: attention softmax of the current denoising queries over the
 *     clean keys, averaged across queries (then 1-D max-pooled, done in the
 *     Python half of the oracle);
 *   - redundancy: Red_j = softmax_j( (1/L_k) sum_i S_ij ), S = cosine similarity
 *     of l2-normalised keys with the diagonal set to zero.
 * Everything is per head; heads never interact.
 *
 * Arrays are head-major and row-contiguous: Q[H][Lq][d], K[H][Lk][d].
 * All arithmetic is IEEE double (compile without -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Rows of queries handled by one independent work item.  The number of row
 * blocks depends only on Lq (not on the thread count), and the per-block
 * partial sums are added in block order, so the result is reproducible. */
#define ORC_ROWS_PER_BLOCK 64

static double dot(const double* a, const double* b, int n) {
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

/*
 * Per-query log-sum-exp of the scaled logits over the clean keys:
 *   lse[h][i] = log sum_j exp(scale * q_i . k_j).
 * (Diagnostic: the normaliser of the importance softmax row i.)
 */
void orc_lse(int H, int Lq, int Lk, int d, double scale,
             const double* Q, const double* K, double* lse) {
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int h = 0; h < H; ++h) {
        for (int i = 0; i < Lq; ++i) {
            const double* q = Q + ((size_t)h * Lq + i) * d;
            const double* Kh = K + (size_t)h * Lk * d;
            double m = -INFINITY;
            for (int j = 0; j < Lk; ++j) {
                double s = scale * dot(q, Kh + (size_t)j * d, d);
                if (s > m) m = s;
            }
            double z = 0.0;
            for (int j = 0; j < Lk; ++j) {
                double s = scale * dot(q, Kh + (size_t)j * d, d);
                z += exp(s - m);
            }
            lse[(size_t)h * Lq + i] = m + log(z);
        }
    }
}

/*
 * Importance before pooling:
 *   P_ij   = exp(s_ij) / sum_k exp(s_ik),  s_ij = scale * q_i . k_j
 *            (row softmax over the clean keys only),
 *   Imp_j  = (1/Lq) sum_i P_ij            (mean across the denoising queries).
 * Each row is computed on its own: logits, row max, row sum, then the
 * normalised row is added into the column accumulator.  No Lq x Lk matrix.
 */
void orc_importance(int H, int Lq, int Lk, int d, double scale,
                    const double* Q, const double* K, double* imp) {
    const int nblk = (Lq + ORC_ROWS_PER_BLOCK - 1) / ORC_ROWS_PER_BLOCK;
    double* part = (double*)calloc((size_t)H * nblk * Lk, sizeof(double));
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)Lk * sizeof(double));
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int h = 0; h < H; ++h) {
            for (int b = 0; b < nblk; ++b) {
                const double* Kh = K + (size_t)h * Lk * d;
                double* acc = part + ((size_t)h * nblk + b) * Lk;
                int i1 = (b + 1) * ORC_ROWS_PER_BLOCK;
                if (i1 > Lq) i1 = Lq;
                for (int i = b * ORC_ROWS_PER_BLOCK; i < i1; ++i) {
                    const double* q = Q + ((size_t)h * Lq + i) * d;
                    double m = -INFINITY;
                    for (int j = 0; j < Lk; ++j) {
                        s[j] = scale * dot(q, Kh + (size_t)j * d, d);
                        if (s[j] > m) m = s[j];
                    }
                    double z = 0.0;
                    for (int j = 0; j < Lk; ++j) {
                        s[j] = exp(s[j] - m);
                        z += s[j];
                    }
                    for (int j = 0; j < Lk; ++j) acc[j] += s[j] / z;
                }
            }
        }
        free(s);
    }
    for (int h = 0; h < H; ++h) {
        double* out = imp + (size_t)h * Lk;
        for (int j = 0; j < Lk; ++j) out[j] = 0.0;
        for (int b = 0; b < nblk; ++b) {
            const double* acc = part + ((size_t)h * nblk + b) * Lk;
            for (int j = 0; j < Lk; ++j) out[j] += acc[j];
        }
        for (int j = 0; j < Lk; ++j) out[j] /= (double)Lq;
    }
    free(part);
}

/* Unit key k_j / max(||k_j||_2, 1e-12): the usual l2 normalisation. */
static void unit_key(const double* k, int d, double* out) {
    double n = sqrt(dot(k, k, d));
    if (n < 1e-12) n = 1e-12;
    for (int c = 0; c < d; ++c) out[c] = k[c] / n;
}

/*
 * Redundancy before its softmax, by the definition (O(Lk^2 d), tiny inputs):
 *   S_ij = khat_i . khat_j for i != j,  S_jj = 0,
 *   r_j  = (1/Lk) sum_i S_ij.
 */
void orc_redundancy_bruteforce(int H, int Lk, int d, const double* K, double* r) {
#pragma omp parallel
    {
        double* kh = (double*)malloc((size_t)Lk * d * sizeof(double));
#pragma omp for schedule(static)
        for (int h = 0; h < H; ++h) {
            const double* Kh = K + (size_t)h * Lk * d;
            for (int j = 0; j < Lk; ++j) unit_key(Kh + (size_t)j * d, d, kh + (size_t)j * d);
            for (int j = 0; j < Lk; ++j) {
                double s = 0.0;
                for (int i = 0; i < Lk; ++i) {
                    double sij = (i == j) ? 0.0 : dot(kh + (size_t)i * d, kh + (size_t)j * d, d);
                    s += sij;
                }
                r[(size_t)h * Lk + j] = s / (double)Lk;
            }
        }
        free(kh);
    }
}

/*
 * The same r_j through the identity sum_{i != j} khat_i . khat_j
 *   = (sum_i khat_i) . khat_j - khat_j . khat_j,
 * so r_j = (u . khat_j - khat_j . khat_j) / Lk with u = sum_i khat_i.
 * (O(Lk d); exact in real arithmetic, equal to the definition up to rounding.)
 */
void orc_redundancy_closed(int H, int Lk, int d, const double* K, double* r) {
#pragma omp parallel
    {
        double* kh = (double*)malloc((size_t)d * sizeof(double));
        double* u = (double*)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(static)
        for (int h = 0; h < H; ++h) {
            const double* Kh = K + (size_t)h * Lk * d;
            for (int c = 0; c < d; ++c) u[c] = 0.0;
            for (int j = 0; j < Lk; ++j) {
                unit_key(Kh + (size_t)j * d, d, kh);
                for (int c = 0; c < d; ++c) u[c] += kh[c];
            }
            for (int j = 0; j < Lk; ++j) {
                unit_key(Kh + (size_t)j * d, d, kh);
                r[(size_t)h * Lk + j] = (dot(u, kh, d) - dot(kh, kh, d)) / (double)Lk;
            }
        }
        free(kh);
        free(u);
    }
}

/* Number of threads the OpenMP runtime will use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
