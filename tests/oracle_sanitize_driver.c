/* Drives every entry point of the C oracle on small seeded problems, for a
 * build with the address and undefined-behaviour sanitizers (host code only;
 * tests/test_oracle_sanitized.py compiles and runs it).  Shapes cover a single
 * token, ragged lengths, dk != dv, every head size, no initial state, each
 * column-block mode and one or more threads; the printed line per shape is
 * what the test counts. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void kda_oracle_gate(const double *z, const double *A, double *g, int64_t B, int64_t T, int64_t H,
                     int64_t dk);
void kda_oracle_forward(const double *q, const double *k, const double *v, const double *g,
                        const double *beta, const double *S0, double *o, double *ST, int64_t B,
                        int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t col_block,
                        int nthreads);
void kda_oracle_decode_step(const double *q, const double *k, const double *v, const double *z,
                            const double *A, const double *beta, double *state, double *o,
                            int64_t N, int64_t H, int64_t dk, int64_t dv);
int kda_oracle_max_threads(void);

static unsigned long long rng = 12345;
static double uni(void) {                 /* xorshift64*, in [-1, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ULL) >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(int64_t n) {
    double *p = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = uni();
    return p;
}

int main(void) {
    static const int64_t shapes[][5] = {   /* B, T, H, dk, dv */
        {1, 1, 1, 32, 32}, {2, 17, 3, 32, 64}, {1, 40, 2, 64, 32}, {3, 5, 1, 128, 128},
        {1, 129, 2, 64, 128}, {2, 3, 4, 128, 32},
    };
    const int nshape = (int)(sizeof shapes / sizeof shapes[0]);
    if (kda_oracle_max_threads() < 1) return 2;
    for (int s = 0; s < nshape; ++s) {
        const int64_t B = shapes[s][0], T = shapes[s][1], H = shapes[s][2];
        const int64_t dk = shapes[s][3], dv = shapes[s][4];
        double *q = arr(B * T * H * dk), *k = arr(B * T * H * dk), *v = arr(B * T * H * dv);
        double *z = arr(B * T * H * dk), *A = arr(H * dk), *beta = arr(B * T * H);
        double *S0 = arr(B * H * dk * dv), *g = arr(B * T * H * dk);
        double *o = arr(B * T * H * dv), *ST = arr(B * H * dk * dv), *od = arr(B * H * dv);
        for (int64_t i = 0; i < B * T * H; ++i) beta[i] = 0.5 * (beta[i] + 1.0);
        kda_oracle_gate(z, A, g, B, T, H, dk);
        for (int mode = 0; mode < 4; ++mode)
            kda_oracle_forward(q, k, v, g, beta, mode == 3 ? NULL : S0, o, ST, B, T, H, dk, dv,
                               mode == 0 ? 0 : (mode == 1 ? 7 : dv), mode == 2 ? 1 : 3);
        kda_oracle_decode_step(q, k, v, z, A, beta, S0, od, B, H, dk, dv);
        printf("shape %d ok %.6g %.6g %.6g\n", s, o[0], ST[0], od[0]);
        free(q); free(k); free(v); free(z); free(A); free(beta);
        free(S0); free(g); free(o); free(ST); free(od);
    }
    return 0;
}
