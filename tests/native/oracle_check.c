/*
 * Drives the C half of the oracle on small random inputs under the host
 * address and undefined-behaviour sanitizers: every row and key loop touches
 * only its arrays, and the checks that pin the oracle still hold:
 *   - sum_j Imp_j = 1 per head (each softmax row sums to 1);
 *   - the closed form of the redundancy equals its brute-force definition;
 *   - Q = 0 gives Imp_j = 1 / L_k (to rounding).
 * Test infrastructure only: it links the oracle, never the library.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void orc_lse(int H, int Lq, int Lk, int d, double scale, const double* Q, const double* K, double* lse);
void orc_importance(int H, int Lq, int Lk, int d, double scale, const double* Q, const double* K, double* imp);
void orc_redundancy_bruteforce(int H, int Lk, int d, const double* K, double* r);
void orc_redundancy_closed(int H, int Lk, int d, const double* K, double* r);

static double uniform(unsigned long long* s) {
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(*s >> 11) / 9007199254740992.0 - 0.5;
}

int main(void) {
    const int H = 3, Lq = 70, Lk = 131, d = 64;
    const double scale = 1.0 / sqrt((double)d);
    double* Q = malloc(sizeof(double) * H * Lq * d);
    double* K = malloc(sizeof(double) * H * Lk * d);
    double* imp = malloc(sizeof(double) * H * Lk);
    double* lse = malloc(sizeof(double) * H * Lq);
    double* rb = malloc(sizeof(double) * H * Lk);
    double* rc = malloc(sizeof(double) * H * Lk);
    if (!Q || !K || !imp || !lse || !rb || !rc) return 2;
    unsigned long long s = 12345;
    for (int i = 0; i < H * Lq * d; ++i) Q[i] = 4.0 * uniform(&s);
    for (int i = 0; i < H * Lk * d; ++i) K[i] = 4.0 * uniform(&s);
    for (int c = 0; c < d; ++c) K[(size_t)(1 * Lk + 5) * d + c] = 0.0;  /* a zero key */
    int fails = 0;
    orc_lse(H, Lq, Lk, d, scale, Q, K, lse);
    orc_importance(H, Lq, Lk, d, scale, Q, K, imp);
    for (int h = 0; h < H; ++h) {
        double t = 0.0;
        for (int j = 0; j < Lk; ++j) t += imp[h * Lk + j];
        if (fabs(t - 1.0) > 1e-12) { printf("head %d: sum of importance %.17g\n", h, t); ++fails; }
    }
    orc_redundancy_bruteforce(H, Lk, d, K, rb);
    orc_redundancy_closed(H, Lk, d, K, rc);
    for (int i = 0; i < H * Lk; ++i)
        if (fabs(rb[i] - rc[i]) > 1e-12) { printf("redundancy %d: %.17g vs %.17g\n", i, rb[i], rc[i]); ++fails; break; }
    for (int i = 0; i < H * Lq * d; ++i) Q[i] = 0.0;
    orc_importance(H, Lq, Lk, d, scale, Q, K, imp);
    for (int i = 0; i < H * Lk; ++i)
        if (fabs(imp[i] * Lk - 1.0) > 1e-12) { printf("Q = 0: Imp %.17g\n", imp[i]); ++fails; break; }
    free(Q); free(K); free(imp); free(lse); free(rb); free(rc);
    printf("%s\n", fails ? "oracle checks failed" : "oracle checks ok");
    return fails != 0;
}
