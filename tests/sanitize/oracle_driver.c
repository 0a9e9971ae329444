/*
 * Runs every entry point of the CPU oracle (oracle/moe_oracle.c) on small
 * seeded layers, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: fp32 and bf16 inputs, top-k with and without
 * renormalisation, k = E, capacity drops, capacity 0, T = 1, a router bias,
 * the residual path and the slots a capacity drop leaves empty. Nothing is
 * compared here (the Python pins do that); the run must end with status 0
 * and no sanitizer report.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_silu(const double *z, int n, double *out);
void orc_logits(const void *x, int xdt, int T, int d, const void *wg, int wdt,
                const float *gate_bias, int E, double *logits);
void orc_route(const double *logits, int T, int E, int k, int renorm, int32_t *idx,
               double *gate, double *prob_sum, double *probs_out);
void orc_permute(const int32_t *idx, int T, int k, int E, int capacity, int32_t *counts,
                 int32_t *offsets, int32_t *dest_row, int32_t *sorted_token);
void orc_expert_rows(const void *x, int xdt, int d, int h, const int32_t *tok, int nrows,
                     const void *w1e, const void *b1e, const void *w2e, const void *b2e, int wdt,
                     double *y);
void orc_combine(const double *y_slots, const int32_t *dest, const double *gate, int ntok, int k,
                 int d, const int32_t *tok, const void *residual, int rdt, double *out);
void orc_aux(const double *prob_sum, const int32_t *counts, int T, int E, double *f, double *P,
             double *loss);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* splitmix64 -> [-1, 1) */
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / (double)(1ull << 52) - 1.0;
}

/* n values in fp32 (dt 0) or as bf16 bit patterns (dt 1), scaled. */
static void *fill(size_t n, int dt, double scale) {
    if (dt == 0) {
        float *a = malloc(n * sizeof *a + 1);
        for (size_t i = 0; i < n; ++i) a[i] = (float)(unif() * scale);
        return a;
    }
    uint16_t *a = malloc(n * sizeof *a + 1);
    for (size_t i = 0; i < n; ++i) {
        float f = (float)(unif() * scale);
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        a[i] = (uint16_t)(u >> 16);
    }
    return a;
}

static void layer(int T, int d, int h, int E, int k, int renorm, int capacity, int dt, int bias,
                  int residual) {
    void *x = fill((size_t)T * d, dt, 1.0);
    void *wg = fill((size_t)E * d, dt, 0.5);
    void *w1 = fill((size_t)E * h * d, dt, 0.3);
    void *b1 = fill((size_t)E * h, dt, 0.1);
    void *w2 = fill((size_t)E * d * h, dt, 0.3);
    void *b2 = fill((size_t)E * d, dt, 0.1);
    float *gb = NULL;
    if (bias) {
        gb = malloc((size_t)E * sizeof *gb);
        for (int e = 0; e < E; ++e) gb[e] = (float)unif();
    }
    const size_t esz = dt == 0 ? 4 : 2;
    double *lg = malloc((size_t)T * E * sizeof *lg);
    orc_logits(x, dt, T, d, wg, dt, gb, E, lg);
    int32_t *idx = malloc((size_t)T * k * sizeof *idx);
    double *gate = malloc((size_t)T * k * sizeof *gate);
    double *ps = malloc((size_t)E * sizeof *ps);
    double *probs = malloc((size_t)T * E * sizeof *probs);
    orc_route(lg, T, E, k, renorm, idx, gate, ps, probs);
    orc_route(lg, T, E, k, renorm, idx, gate, ps, NULL);
    int32_t *counts = malloc((size_t)E * sizeof *counts);
    int32_t *offsets = malloc((size_t)(E + 1) * sizeof *offsets);
    int32_t *dest = malloc((size_t)T * k * sizeof *dest);
    int32_t *st = malloc((size_t)T * k * sizeof *st + 4);
    orc_permute(idx, T, k, E, capacity, counts, offsets, dest, st);
    /* every slot's expert output, as the Python oracle assembles them */
    double *y_slots = calloc((size_t)T * k * d, sizeof *y_slots);
    for (int e = 0; e < E; ++e) {
        const int r0 = offsets[e], n = offsets[e + 1] - offsets[e];
        double *y = malloc(((size_t)n * d + 1) * sizeof *y);
        orc_expert_rows(x, dt, d, h, st + r0, n, (const char *)w1 + (size_t)e * h * d * esz,
                        (const char *)b1 + (size_t)e * h * esz,
                        (const char *)w2 + (size_t)e * d * h * esz,
                        (const char *)b2 + (size_t)e * d * esz, dt, y);
        for (int i = 0; i < T * k; ++i)
            if (dest[i] >= r0 && dest[i] < r0 + n)
                memcpy(y_slots + (size_t)i * d, y + (size_t)(dest[i] - r0) * d, d * sizeof *y);
        free(y);
    }
    int32_t *tok = malloc((size_t)T * sizeof *tok);
    for (int t = 0; t < T; ++t) tok[t] = t;
    double *out = malloc((size_t)T * d * sizeof *out);
    orc_combine(y_slots, dest, gate, T, k, d, tok, residual ? x : NULL, dt, out);
    double *f = malloc((size_t)E * sizeof *f), *P = malloc((size_t)E * sizeof *P), loss;
    orc_aux(ps, counts, T, E, f, P, &loss);
    double z[5] = {-40.0, -1.5, 0.0, 2.0, 700.0}, sz[5];
    orc_silu(z, 5, sz);
    printf("T=%d d=%d h=%d E=%d k=%d renorm=%d cap=%d dt=%d bias=%d res=%d: rows %d loss %.6f\n",
           T, d, h, E, k, renorm, capacity, dt, bias, residual, offsets[E], loss);
    free(x); free(wg); free(w1); free(b1); free(w2); free(b2); free(gb); free(lg); free(idx);
    free(gate); free(ps); free(probs); free(counts); free(offsets); free(dest); free(st);
    free(y_slots); free(tok); free(out); free(f); free(P);
}

int main(void) {
    layer(9, 8, 12, 4, 2, 1, -1, 0, 0, 0);
    layer(9, 8, 12, 4, 2, 1, -1, 1, 1, 1);
    layer(16, 6, 10, 5, 1, 0, 2, 1, 1, 1);  /* capacity drops */
    layer(7, 4, 6, 3, 3, 1, -1, 0, 0, 1);   /* k = E */
    layer(5, 4, 6, 3, 2, 1, 0, 1, 0, 1);    /* capacity 0: every slot dropped */
    layer(1, 8, 8, 6, 2, 0, 1, 0, 1, 0);    /* one token */
    layer(33, 16, 24, 8, 4, 1, 5, 1, 1, 0);
    return 0;
}
