/* Drives every entry point of the CPU oracle (oracle/lq_oracle.c, compiled
 * into the same executable) on small seeded inputs and the degenerate cases
 * (empty runs, no compensators, a window of one token, all-zero states, both
 * gates, both code formats, the binary16 buffer), so that AddressSanitizer and
 * UndefinedBehaviorSanitizer see all of its loops.  Test infrastructure:
 * built and run by tests/test_sanitizers.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_recurrence(int, int, int, int, int, double*, const float*, const float*, const float*,
                   const float*, const float*, double*);
int orc_qz(int, int, int, int, int, int, const double*, const int*, int8_t*, float*, float*, int*,
           float*, double*, double*);
int orc_dequant(int, int, int, int, int, const int8_t*, const float*, const float*, const int*,
                const float*, double*);
int orc_replay_output(int, int, int, int, int, int, int, const int8_t*, const float*, const float*,
                      const int*, const float*, const float*, const float*, const float*, const float*,
                      const float*, double*);
int orc_windowed_run(int, int, int, int, int, int, int, int, int, int, const double*, const float*,
                     const float*, const float*, const float*, const float*, const int*, double*, double*);
double orc_e4m3_value(int);
int orc_e4m3_encode(double);
float orc_fp16_round(float);

static uint64_t rng_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}
static float* fill(size_t n, double lo, double hi) {
    float* p = malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * urand());
    return p;
}

static int run_case(int fmt, int buf16, int U, int d, int T, int gate_kind, int W, int n_c, int smooth,
                    int zero_state) {
    const int g = gate_kind ? d : 1;
    const int D = d;
    size_t SS = (size_t)U * d * d;
    double* S0 = calloc(SS ? SS : 1, sizeof(double));
    if (!zero_state)
        for (size_t i = 0; i < SS; ++i) S0[i] = 4.0 * urand() - 2.0;
    float* q = fill((size_t)T * U * d, -1, 1);
    float* k = fill((size_t)T * U * d, -1, 1);
    float* v = fill((size_t)T * U * d, -3, 3);
    float* b = fill((size_t)T * U, 0, 1);
    float* a = fill((size_t)T * U * g, 0.85, 1.0);
    int* force = malloc(sizeof(int) * (size_t)(U ? U : 1));
    for (int u = 0; u < U; ++u) force[u] = (u % 3 == 1) ? T / 2 : -1;
    double* o = malloc(sizeof(double) * ((size_t)(T > 0 ? T : 1) * U * d + 1)); /* also the replay output [U][d] */
    double* Sout = malloc(sizeof(double) * (SS + 1));
    int rc = 0;
    rc |= orc_windowed_run(fmt, buf16, U, d, d, T, gate_kind, W, n_c, smooth, S0, q, k, v, b, a, force, o, Sout);
    double* S = malloc(sizeof(double) * (SS + 1));
    for (size_t i = 0; i < SS; ++i) S[i] = S0[i];
    rc |= orc_recurrence(U, d, d, T, gate_kind, S, q, k, v, b, a, o);
    int8_t* codes = malloc(SS + 1);
    float* sg = malloc(sizeof(float) * ((size_t)U * d + 1));
    float* sm = malloc(sizeof(float) * ((size_t)U * d + 1));
    int* ci = malloc(sizeof(int) * ((size_t)U * n_c + 1));
    float* cv = malloc(sizeof(float) * ((size_t)U * n_c * D + 1));
    double* x = malloc(sizeof(double) * (SS + 1));
    double* sc = malloc(sizeof(double) * ((size_t)U * 2 * d + 1));
    rc |= orc_qz(fmt, U, d, d, n_c, smooth, S, NULL, codes, sg, sm, ci, cv, x, sc);
    rc |= orc_dequant(fmt, U, d, d, n_c, codes, sg, sm, ci, cv, S);
    /* the buffered replay over min(T, W) entries, unit-major */
    const int n = T < W ? T : W;
    float* qu = fill((size_t)U * d, -1, 1); /* one query per unit */
    rc |= orc_replay_output(fmt, U, d, d, n_c, gate_kind, n, codes, sg, sm, ci, cv, k, v, b, a, qu, o);
    free(qu);
    free(S0); free(q); free(k); free(v); free(b); free(a); free(force); free(o); free(Sout);
    free(S); free(codes); free(sg); free(sm); free(ci); free(cv); free(x); free(sc);
    return rc;
}

int main(void) {
    int rc = 0, cases = 0;
    for (int fmt = 0; fmt < 2; ++fmt)
        for (int gk = 0; gk < 2; ++gk)
            for (int buf16 = 0; buf16 < 2; ++buf16) {
                rc |= run_case(fmt, buf16, 3, 8, 19, gk, 5, 2, 1, 0); ++cases;
                rc |= run_case(fmt, buf16, 2, 16, 9, gk, 1, 0, 0, 0); ++cases;  /* naive per-token */
                rc |= run_case(fmt, buf16, 2, 4, 12, gk, 4, 8, 1, 1); ++cases;  /* zero state, all lines */
                rc |= run_case(fmt, buf16, 1, 8, 0, gk, 3, 1, 1, 0); ++cases;   /* no tokens */
                rc |= run_case(fmt, buf16, 0, 8, 4, gk, 3, 1, 1, 0); ++cases;   /* no units */
            }
    /* the two 8-bit/16-bit formats over their whole ranges */
    for (int c = 0; c < 256; ++c) {
        double val = orc_e4m3_value(c);
        if (!isnan(val) && orc_e4m3_value(orc_e4m3_encode(val)) != val) rc |= 1;
    }
    for (int i = -70000; i <= 70000; i += 7) (void)orc_fp16_round((float)i * 0.37f);
    (void)orc_fp16_round(NAN);
    (void)orc_e4m3_encode(1e30);
    if (rc) {
        fprintf(stderr, "an oracle call returned an error\n");
        return 1;
    }
    printf("oracle driver: %d cases, all calls returned 0\n", cases);
    return 0;
}
