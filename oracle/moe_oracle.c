/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the forward pass of
 * one Mixture-of-Experts layer, used to check the GPU library. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the GPU path.
 *
 * Every sum is accumulated in double from the exact input values (bf16
 * inputs are widened exactly; fp32 inputs are widened exactly). Loops run in
 * the order the definitions are written; OpenMP only splits independent
 * outputs between threads, never a sum.
 *
 * Sources (the pages this follows):
 *   [P5] "MoE混合专家模型路由机制原理与稀疏激活实现" (MoE routing mechanism and
 *        sparse activation), yunthe.com:
 *        - section "MoE混合专家模型架构与门控路由原理": gate equation
 *          G(x) = softmax(TopK(x . W_g)) and output y = sum_i G(x)_i E_i(x);
 *        - section "Top-K门控路由的PyTorch实现": TopKRouter (linear gate
 *          without bias, softmax over experts, top-k, renormalise), Expert
 *          (w2(silu(w1 x)) with nn.Linear biases), MoELayer (slot-by-slot
 *          weighted accumulation), load_balancing_loss (E * sum f*P);
 *        - section "Expert Choice路由策略与容量因子调优": capacity
 *          = tokens / experts * capacity_factor, rejected tokens pass on the
 *          residual connection.
 *   [P3] "MoE 架构完整指南：路由、负载均衡、EP、训练稳定性、Serving"
 *        (walkerchi.com), section 5.2: a per-expert router bias added to
 *        the logits.
 *
 * Readings where the pages are silent (each is listed with its reason in
 * the design notes of the repository):
 *   - top-k ties: the lower expert index wins; comparison is IEEE ">" so
 *     +0 and -0 are equal;
 *   - selection is made on the logits (monotone-equal to selecting on the
 *     softmax probabilities);
 *   - renorm = 0 gives the gate as the full-softmax probability (Switch
 *     style top-1); renorm = 1 renormalises over the selected k;
 *   - capacity < 0 means unlimited; capacity >= 0 keeps, per expert, the
 *     first `capacity` assignments in ascending flat order t*k + j;
 *   - P (token share) counts assignments before any capacity drop and is
 *     divided by T.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Exact widening of one stored element to double. */
static double widen(const void *p, int dtype, size_t i) {
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))   [P5, Expert.forward]. */
static double silu(double z) { return z / (1.0 + exp(-z)); }

void orc_silu(const double *z, int n, double *out) {
    for (int i = 0; i < n; ++i) out[i] = silu(z[i]);
}

/*
 * Router logits  l[t,e] = sum_i x[t,i] * W_g[e,i]  (+ b_g[e] when given).
 * [P5] TopKRouter: nn.Linear(dim, E, bias=False); [P3] 5.2: router bias.
 */
void orc_logits(const void *x, int xdt, int T, int d, const void *wg, int wdt,
                const float *gate_bias, int E, double *logits) {
    double *w = (double *)malloc(sizeof(double) * (size_t)E * d);
    for (size_t i = 0; i < (size_t)E * d; ++i) w[i] = widen(wg, wdt, i);
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double *xr = (double *)malloc(sizeof(double) * (size_t)d);
        for (int i = 0; i < d; ++i) xr[i] = widen(x, xdt, (size_t)t * d + i);
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += xr[i] * w[(size_t)e * d + i];
            if (gate_bias) s += (double)gate_bias[e];
            logits[(size_t)t * E + e] = s;
        }
        free(xr);
    }
    free(w);
}

/*
 * Routing from given logits.
 *   selection: the k experts with the largest logits, lower index first on
 *              equal values (repeated arg-max over the not-yet-chosen);
 *   probs:     p[t,e] = exp(l - max) / sum_e' exp(l_e' - max);
 *   gates:     renorm: p[t,S_j] / sum_{S} p   [P5, TopKRouter.forward]
 *              else:   p[t,S_j];
 *   prob_sum:  sum over t of p[t,e], t ascending (input to f of the aux loss).
 * probs_out may be NULL; otherwise it receives p [T][E].
 */
void orc_route(const double *logits, int T, int E, int k, int renorm,
               int32_t *idx, double *gate, double *prob_sum, double *probs_out) {
    double *probs = probs_out ? probs_out : (double *)malloc(sizeof(double) * (size_t)T * E);
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double *p = probs + (size_t)t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * k + j] = best;
        }
        free(taken);
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) z += exp(l[e] - m);
        for (int e = 0; e < E; ++e) p[e] = exp(l[e] - m) / z;
        double sel = 0.0;
        for (int j = 0; j < k; ++j) sel += p[idx[(size_t)t * k + j]];
        for (int j = 0; j < k; ++j) {
            double pj = p[idx[(size_t)t * k + j]];
            gate[(size_t)t * k + j] = renorm ? pj / sel : pj;
        }
    }
    if (prob_sum) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int t = 0; t < T; ++t) s += probs[(size_t)t * E + e];
            prob_sum[e] = s;
        }
    }
    if (!probs_out) free(probs);
}

/*
 * Dispatch bookkeeping (counting sort by expert with capacity).
 *   counts[e]   = #{(t,j) : idx[t,j] == e}           (before any drop)
 *   kept[e]     = counts[e] if capacity < 0 else min(counts[e], capacity)
 *   offsets     = exclusive prefix sum of kept, offsets[E] = R
 *   dest_row    = offsets[e] + (rank of (t,j) among expert e's assignments
 *                 in ascending t*k+j) when that rank < kept[e], else -1
 *   sorted_token[dest_row[t,j]] = t
 * Capacity and the residual pass-through: [P5] "Expert Choice路由策略与容量因子调优".
 */
void orc_permute(const int32_t *idx, int T, int k, int E, int capacity,
                 int32_t *counts, int32_t *offsets, int32_t *dest_row,
                 int32_t *sorted_token) {
    const long n = (long)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long f = 0; f < n; ++f) counts[idx[f]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int kept = counts[e];
        if (capacity >= 0 && kept > capacity) kept = capacity;
        offsets[e + 1] = offsets[e] + kept;
    }
    for (int e = 0; e < E; ++e) {
        int kept = offsets[e + 1] - offsets[e];
        int rank = 0;
        for (long f = 0; f < n; ++f) {
            if (idx[f] != e) continue;
            if (rank < kept) {
                int r = offsets[e] + rank;
                dest_row[f] = r;
                sorted_token[r] = (int32_t)(f / k);
            } else {
                dest_row[f] = -1;
            }
            ++rank;
        }
    }
}

/*
 * One expert applied to a list of token rows   [P5, Expert]:
 *   z[r,n]  = sum_i W1[n,i] * x[tok_r, i] + b1[n]       W1 is [h][d]
 *   a[r,n]  = SiLU(z[r,n])
 *   y[r,m]  = sum_n W2[m,n] * a[r,n] + b2[m]            W2 is [d][h]
 * w1e/b1e/w2e/b2e point at this expert's slices; biases may be NULL.
 * x has row stride d. y is [nrows][d] double.
 */
void orc_expert_rows(const void *x, int xdt, int d, int h, const int32_t *tok,
                     int nrows, const void *w1e, const void *b1e,
                     const void *w2e, const void *b2e, int wdt, double *y) {
    if (nrows <= 0) return;
    double *a = (double *)malloc(sizeof(double) * (size_t)nrows * h);
    double *xr = (double *)malloc(sizeof(double) * (size_t)nrows * d);
    for (int r = 0; r < nrows; ++r)
        for (int i = 0; i < d; ++i)
            xr[(size_t)r * d + i] = widen(x, xdt, (size_t)tok[r] * d + i);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < h; ++n) {
        double *w = (double *)malloc(sizeof(double) * (size_t)d);
        for (int i = 0; i < d; ++i) w[i] = widen(w1e, wdt, (size_t)n * d + i);
        double b = b1e ? widen(b1e, wdt, (size_t)n) : 0.0;
        for (int r = 0; r < nrows; ++r) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += w[i] * xr[(size_t)r * d + i];
            a[(size_t)r * h + n] = silu(s + b);
        }
        free(w);
    }
#pragma omp parallel for schedule(static)
    for (int m = 0; m < d; ++m) {
        double *w = (double *)malloc(sizeof(double) * (size_t)h);
        for (int n = 0; n < h; ++n) w[n] = widen(w2e, wdt, (size_t)m * h + n);
        double b = b2e ? widen(b2e, wdt, (size_t)m) : 0.0;
        for (int r = 0; r < nrows; ++r) {
            double s = 0.0;
            for (int n = 0; n < h; ++n) s += w[n] * a[(size_t)r * h + n];
            y[(size_t)r * d + m] = s + b;
        }
        free(w);
    }
    free(xr);
    free(a);
}

/*
 * Combine for a list of tokens   [P5, gate-weighted output and MoELayer]:
 *   out[t] = (residual ? residual[t] : 0) + sum_{j kept} gate[t,j] * y[t,j]
 * summed over j ascending. y_slots is [ntok][k][d] (rows of dropped slots
 * are ignored), dest is [ntok][k] with -1 for a dropped slot, gate [ntok][k].
 * residual (row stride d, given dtype) is indexed by tok[i]; may be NULL.
 */
void orc_combine(const double *y_slots, const int32_t *dest, const double *gate,
                 int ntok, int k, int d, const int32_t *tok, const void *residual,
                 int rdt, double *out) {
#pragma omp parallel for schedule(static)
    for (int i = 0; i < ntok; ++i) {
        for (int m = 0; m < d; ++m) {
            double s = residual ? widen(residual, rdt, (size_t)tok[i] * d + m) : 0.0;
            for (int j = 0; j < k; ++j) {
                if (dest[(size_t)i * k + j] < 0) continue;
                s += gate[(size_t)i * k + j] * y_slots[((size_t)i * k + j) * d + m];
            }
            out[(size_t)i * d + m] = s;
        }
    }
}

/*
 * Load-balancing auxiliary loss   [P5, load_balancing_loss]:
 *   f[e] = prob_sum[e] / T   (mean full-softmax probability)
 *   P[e] = counts[e] / T     (top-k assignments per token, before drops)
 *   loss = E * sum_e f[e] * P[e]
 */
void orc_aux(const double *prob_sum, const int32_t *counts, int T, int E,
             double *f, double *P, double *loss) {
    double s = 0.0;
    for (int e = 0; e < E; ++e) {
        f[e] = prob_sum[e] / (double)T;
        P[e] = (double)counts[e] / (double)T;
        s += f[e] * P[e];
    }
    *loss = (double)E * s;
}
