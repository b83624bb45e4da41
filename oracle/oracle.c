/*
 * oracle.c -- plain, slow CPU reference of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. It shares no code
 * with the HIP library. Built with -ffp-contract=off so that no multiply-add
 * is fused behind the source's back; the only fused operations are the
 * explicit fmaf calls of the router definition.
 *
 * Pins (what the tests check this file against) are listed in each
 * function's header comment in oracle.h and in tests/test_oracle_*.py.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* bf16 is the upper 16 bits of a binary32: widening is exact. */
static inline float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static inline float load_f(const void* p, int xtype, size_t i)
{
    if (xtype == 1)
        return bf16_bits_to_float(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

/* ------------------------------------------------------------------ router */

int oracle_route(const void* x, const void* w, int xtype, const float* bias,
                 int64_t T, int d, int E, int k, int renorm,
                 float* logits, int32_t* idx, double* gates)
{
    if (!x || !w || !logits || !idx || !gates) return -1;
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return -1;
    if (xtype != 0 && xtype != 1) return -1;

    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        float* l = logits + (size_t)t * E;
        /* scores: one fused multiply-add per term, i ascending, from +0 */
        for (int e = 0; e < E; ++e) l[e] = 0.0f;
        for (int i = 0; i < d; ++i) {
            float xi = load_f(x, xtype, (size_t)t * d + i);
            for (int e = 0; e < E; ++e)
                l[e] = fmaf(xi, load_f(w, xtype, (size_t)i * E + e), l[e]);
        }
        if (bias)
            for (int e = 0; e < E; ++e) l[e] = l[e] + bias[e];
        for (int e = 0; e < E; ++e)
            if (!isfinite(l[e])) bad = 1;

        /* top-k: k rounds of "largest remaining"; a strict comparison keeps
         * the lowest index among equal values (and -0 == +0) */
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        int32_t* id = idx + (size_t)t * k;
        for (int s = 0; s < k; ++s) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            id[s] = best;
        }
        free(taken);

        /* router weights: softmax restricted to the chosen experts (renorm)
         * or the full softmax probability of each chosen expert */
        double m = (double)l[id[0]];
        double* g = gates + (size_t)t * k;
        double denom = 0.0;
        for (int s = 0; s < k; ++s) {
            g[s] = exp((double)l[id[s]] - m);
            denom += g[s];
        }
        if (!renorm) {
            denom = 0.0;
            for (int e = 0; e < E; ++e) denom += exp((double)l[e] - m);
        }
        for (int s = 0; s < k; ++s) g[s] = g[s] / denom;
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------- permutation */

/* Shared by both packings: expert e's region receives, in ascending flat
 * order, every assignment whose key is e. Written as one pass per expert so
 * that it reads like the definition (for each expert: find its assignments,
 * copy them into its slice of the packed buffer). */
static void pack_by_key(const int32_t* key, int64_t n, int E,
                        int32_t* counts, int32_t* offsets,
                        int32_t* perm_src, int32_t* dest)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < n; ++a) counts[key[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int e = 0; e < E; ++e) {
        int64_t j = offsets[e];
        for (int64_t a = 0; a < n; ++a) {
            if (key[a] != e) continue;
            perm_src[j] = (int32_t)a;
            dest[a] = (int32_t)j;
            ++j;
        }
    }
}

int oracle_permute(const int32_t* idx, int64_t TK, int E,
                   int32_t* counts, int32_t* offsets,
                   int32_t* perm_src, int32_t* dest)
{
    if (!idx || !counts || !offsets || !perm_src || !dest) return -1;
    if (TK < 0 || E <= 0 || TK > INT32_MAX) return -1;
    for (int64_t a = 0; a < TK; ++a)
        if (idx[a] < 0 || idx[a] >= E) return -2;
    pack_by_key(idx, TK, E, counts, offsets, perm_src, dest);
    return 0;
}

int oracle_permute_capacity(const int32_t* idx, int64_t TK, int E, int64_t capacity,
                            int32_t* routed, int32_t* counts, int32_t* offsets,
                            int32_t* perm_src, int32_t* dest)
{
    if (!idx || !routed || !counts || !offsets || !perm_src || !dest) return -1;
    if (TK < 0 || E <= 0 || TK > INT32_MAX || capacity < 0) return -1;
    for (int64_t a = 0; a < TK; ++a)
        if (idx[a] < 0 || idx[a] >= E) return -2;
    for (int e = 0; e < E; ++e) routed[e] = 0;
    for (int64_t a = 0; a < TK; ++a) routed[idx[a]] += 1;
    for (int e = 0; e < E; ++e) counts[e] = routed[e] < capacity ? routed[e] : (int32_t)capacity;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t a = 0; a < TK; ++a) dest[a] = -1;
    /* for each expert: its assignments in ascending a, the first `capacity`
     * of them into its slice of the packed buffer */
    for (int e = 0; e < E; ++e) {
        int64_t j = offsets[e];
        int64_t kept = 0;
        for (int64_t a = 0; a < TK && kept < counts[e]; ++a) {
            if (idx[a] != e) continue;
            perm_src[j] = (int32_t)a;
            dest[a] = (int32_t)j;
            ++j;
            ++kept;
        }
    }
    return 0;
}

int oracle_permute_range(const int32_t* idx, int64_t TK, int e_first, int E_loc,
                         int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* dest)
{
    if (!idx || !counts || !offsets || !perm_src || !dest) return -1;
    if (TK < 0 || TK > INT32_MAX || E_loc <= 0 || e_first < 0) return -1;
    for (int e = 0; e < E_loc; ++e) counts[e] = 0;
    for (int64_t a = 0; a < TK; ++a) {
        int64_t l = (int64_t)idx[a] - e_first;
        if (l >= 0 && l < E_loc) counts[l] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E_loc; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t a = 0; a < TK; ++a) dest[a] = -1;
    /* for each local expert: its assignments in ascending a, into its slice */
    for (int e = 0; e < E_loc; ++e) {
        int64_t j = offsets[e];
        for (int64_t a = 0; a < TK; ++a) {
            if ((int64_t)idx[a] - e_first != e) continue;
            perm_src[j] = (int32_t)a;
            dest[a] = (int32_t)j;
            ++j;
        }
    }
    return 0;
}

int oracle_permute_recv(const int32_t* recv, int S, int E_loc, int64_t N,
                        int32_t* counts, int32_t* offsets,
                        int32_t* perm_src, int32_t* dest)
{
    if (!recv || !counts || !offsets || !perm_src || !dest) return -1;
    if (S <= 0 || E_loc <= 0 || N < 0 || N > INT32_MAX) return -1;
    int64_t total = 0;
    for (int c = 0; c < S * E_loc; ++c) {
        if (recv[c] < 0) return -2;
        total += recv[c];
    }
    if (total != N) return -2;
    /* the local expert of every received row, in arrival order:
     * sender 0's rows for expert 0, 1, ..., then sender 1's, ... */
    int32_t* key = (int32_t*)malloc((size_t)(N > 0 ? N : 1) * sizeof(int32_t));
    if (!key) return -1;
    int64_t r = 0;
    for (int i = 0; i < S; ++i)
        for (int j = 0; j < E_loc; ++j)
            for (int32_t q = 0; q < recv[i * E_loc + j]; ++q) key[r++] = j;
    pack_by_key(key, N, E_loc, counts, offsets, perm_src, dest);
    free(key);
    return 0;
}

int oracle_gather(const void* x, int elem_bytes, int64_t d,
                  const int32_t* perm_src, int64_t rows, int k, void* x_perm)
{
    if (!x || !perm_src || !x_perm || elem_bytes <= 0 || d <= 0 || k <= 0) return -1;
    size_t rb = (size_t)d * (size_t)elem_bytes;
    for (int64_t j = 0; j < rows; ++j) {
        int64_t t = perm_src[j] / k;
        memcpy((char*)x_perm + (size_t)j * rb, (const char*)x + (size_t)t * rb, rb);
    }
    return 0;
}

/* -------------------------------------------------------------- expert FFN */

/* The value of v rounded once to bf16 (8 significant bits, to nearest, ties
 * to even), straight from double: v = m 2^ex with m in [0.5, 1), so the bf16
 * grid around v has spacing 2^(ex - 8). bf16 shares float32's exponent range:
 * below its smallest normal 2^-126 (ex < -125) the grid is the subnormal one,
 * of fixed spacing 2^-133. */
static double round_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int ex = 0;
    (void)frexp(v, &ex);
    if (ex < -125) ex = -125;
    return ldexp(nearbyint(ldexp(v, 8 - ex)), ex - 8);
}

int oracle_round_bf16(double* a, int64_t n)
{
    if (!a || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) a[i] = round_bf16(a[i]);
    return 0;
}

int oracle_expert_ffn_rows(const void* x, int xtype, int64_t N, int d, int f, int E,
                           const int32_t* offsets,
                           const void* wg, const void* wv, const void* wo,
                           const int64_t* rows, int64_t nrows, int x_compact, double* y)
{
    return oracle_expert_ffn_rows_h(x, xtype, N, d, f, E, offsets, wg, wv, wo, rows, nrows,
                                    x_compact, 0, y);
}

int oracle_expert_ffn_rows_h(const void* x, int xtype, int64_t N, int d, int f, int E,
                             const int32_t* offsets,
                             const void* wg, const void* wv, const void* wo,
                             const int64_t* rows, int64_t nrows, int x_compact, int h_bf16,
                             double* y)
{
    if (!x || !offsets || !wg || !wv || !wo || !rows || !y) return -1;
    if (d <= 0 || f <= 0 || E <= 0 || N < 0) return -1;
    if (offsets[0] != 0 || offsets[E] != N) return -2;
    for (int e = 0; e < E; ++e)
        if (offsets[e + 1] < offsets[e]) return -2;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return -2;

#pragma omp parallel
    {
        double* g = (double*)malloc(sizeof(double) * (size_t)f);
        double* v = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t j = rows[r];
            int64_t xr = x_compact ? r : j;
            int e = 0;
            while (!(offsets[e] <= j && j < offsets[e + 1])) ++e;
            size_t wbase = (size_t)e * (size_t)d * (size_t)f;
            for (int c = 0; c < f; ++c) { g[c] = 0.0; v[c] = 0.0; }
            for (int i = 0; i < d; ++i) {
                double xi = (double)load_f(x, xtype, (size_t)xr * d + i);
                size_t wrow = wbase + (size_t)i * f;
                for (int c = 0; c < f; ++c) {
                    g[c] += xi * (double)load_f(wg, xtype, wrow + c);
                    v[c] += xi * (double)load_f(wv, xtype, wrow + c);
                }
            }
            /* SwiGLU: silu(g) * v, silu(z) = z * sigmoid(z) */
            for (int c = 0; c < f; ++c) g[c] = g[c] / (1.0 + exp(-g[c])) * v[c];
            /* h stored in bf16 between the two products (the storage point of
             * bf16 data with fp32 accumulation), when asked */
            if (h_bf16)
                for (int c = 0; c < f; ++c) g[c] = round_bf16(g[c]);
            double* yo = y + (size_t)r * d;
            for (int o = 0; o < d; ++o) yo[o] = 0.0;
            for (int c = 0; c < f; ++c) {
                double hc = g[c];
                size_t wrow = wbase + (size_t)c * d;
                for (int o = 0; o < d; ++o) yo[o] += hc * (double)load_f(wo, xtype, wrow + o);
            }
        }
        free(g);
        free(v);
    }
    return 0;
}

/* ----------------------------------------------------------------- combine */

int oracle_combine(const int32_t* tokens, int64_t ntok, int k, int64_t d,
                   const int32_t* dest, const double* gates,
                   const double* y, const int64_t* yrow,
                   const double* shared, double* out)
{
    if (!tokens || !dest || !y || !out || k <= 0 || d <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < ntok; ++r) {
        int64_t t = tokens[r];
        double* o = out + (size_t)r * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int s = 0; s < k; ++s) {
            int64_t a = t * k + s;
            int64_t j = dest[a];
            if (j < 0) continue;   /* dropped by a capacity: contributes nothing */
            int64_t row = yrow ? yrow[j] : j;
            if (row < 0) { bad = 1; continue; }
            double gw = gates ? gates[a] : 1.0;
            const double* yr = y + (size_t)row * d;
            for (int64_t c = 0; c < d; ++c) o[c] += gw * yr[c];
        }
        if (shared) {
            const double* sr = shared + (size_t)r * d;
            for (int64_t c = 0; c < d; ++c) o[c] += sr[c];
        }
    }
    return bad ? -3 : 0;
}

/* ---------------------------------------------------------------- backward
 *
 * The gradients of a scalar loss through the layer, by the chain rule on the
 * definitions above, in double. The selection (top-k ids, packing) is
 * piecewise constant in its inputs and passes no gradient; everything else
 * is differentiated as written.
 */

int oracle_route_backward(const float* logits, const int32_t* idx, const double* gates,
                          const double* d_gates, int64_t T, int E, int k, int renorm,
                          double* d_logits)
{
    if (!logits || !idx || !gates || !d_gates || !d_logits) return -1;
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const int32_t* id = idx + (size_t)t * k;
        const double* g = gates + (size_t)t * k;
        const double* dg = d_gates + (size_t)t * k;
        double* dl = d_logits + (size_t)t * E;
        /* sum over the selected of g * dg: the part every logit shares */
        double gdg = 0.0;
        for (int s = 0; s < k; ++s) gdg += g[s] * dg[s];
        for (int e = 0; e < E; ++e) dl[e] = 0.0;
        if (renorm) {
            /* g_s = exp(l_{e_s}) / sum_r exp(l_{e_r}):
             * dg_s/dl_{e_r} = g_s (delta_sr - g_r) */
            for (int s = 0; s < k; ++s) dl[id[s]] = g[s] * (dg[s] - gdg);
        } else {
            /* g_s = p_{e_s}, p = softmax over all E: dp_a/dl_b = p_a (delta_ab - p_b) */
            const float* l = logits + (size_t)t * E;
            double m = (double)l[id[0]];
            double denom = 0.0;
            for (int e = 0; e < E; ++e) denom += exp((double)l[e] - m);
            for (int e = 0; e < E; ++e) dl[e] = -(exp((double)l[e] - m) / denom) * gdg;
            for (int s = 0; s < k; ++s) dl[id[s]] += g[s] * dg[s];
        }
    }
    return 0;
}

int oracle_router_grads(const void* x, const void* w, int xtype, int64_t T, int d, int E,
                        const double* d_logits, const int32_t* tokens, int64_t ntok,
                        double* d_x, double* d_w)
{
    if (!x || !w || !d_logits || d <= 0 || E <= 0 || T < 0) return -1;
    if (d_x) {
        if (!tokens) return -1;
        /* d_x[r,i] = sum_e d_logits[t,e] W_r[i,e] */
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < ntok; ++r) {
            int64_t t = tokens[r];
            const double* dl = d_logits + (size_t)t * E;
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int e = 0; e < E; ++e) acc += dl[e] * (double)load_f(w, xtype, (size_t)i * E + e);
                d_x[(size_t)r * d + i] = acc;
            }
        }
    }
    if (d_w) {
        /* d_w[i,e] = sum_t x[t,i] d_logits[t,e] */
#pragma omp parallel for schedule(static)
        for (int i = 0; i < d; ++i) {
            double* o = d_w + (size_t)i * E;
            for (int e = 0; e < E; ++e) o[e] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                double xi = (double)load_f(x, xtype, (size_t)t * d + i);
                const double* dl = d_logits + (size_t)t * E;
                for (int e = 0; e < E; ++e) o[e] += xi * dl[e];
            }
        }
    }
    return 0;
}

int oracle_combine_backward_gates(const int32_t* tokens, int64_t ntok, int k, int64_t d,
                                  const int32_t* dest, const double* y, const int64_t* yrow,
                                  const double* d_out, double* d_gates)
{
    if (!tokens || !dest || !y || !d_out || !d_gates || k <= 0 || d <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < ntok; ++r) {
        int64_t t = tokens[r];
        const double* go = d_out + (size_t)r * d;
        for (int s = 0; s < k; ++s) {
            int64_t j = dest[t * k + s];
            double acc = 0.0;
            if (j >= 0) {
                int64_t row = yrow ? yrow[j] : j;
                if (row < 0) { bad = 1; continue; }
                const double* yr = y + (size_t)row * d;
                for (int64_t c = 0; c < d; ++c) acc += go[c] * yr[c];
            }
            d_gates[(size_t)r * k + s] = acc;
        }
    }
    return bad ? -3 : 0;
}

int oracle_combine_backward_rows(const int32_t* perm_src, const int64_t* rows, int64_t nrows,
                                 int k, int64_t d, const double* gates, const double* d_out,
                                 double* d_y)
{
    if (!perm_src || !rows || !d_out || !d_y || k <= 0 || d <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t a = perm_src[rows[r]];
        double gw = gates ? gates[a] : 1.0;
        const double* go = d_out + (size_t)(a / k) * d;
        for (int64_t c = 0; c < d; ++c) d_y[(size_t)r * d + c] = gw * go[c];
    }
    return 0;
}

/* expert of packed row j */
static int expert_of(const int32_t* offsets, int E, int64_t j)
{
    int e = 0;
    while (e < E && !(offsets[e] <= j && j < offsets[e + 1])) ++e;
    return e;
}

int oracle_expert_ffn_backward_rows(const void* x, int xtype, int64_t N, int d, int f, int E,
                                    const int32_t* offsets,
                                    const void* wg, const void* wv, const void* wo,
                                    const int64_t* rows, int64_t nrows, int x_compact,
                                    const double* d_y, double* act, double* d_act, double* d_x)
{
    return oracle_expert_ffn_backward_rows_h(x, xtype, N, d, f, E, offsets, wg, wv, wo, rows,
                                             nrows, x_compact, 0, d_y, act, d_act, d_x);
}

int oracle_expert_ffn_backward_rows_h(const void* x, int xtype, int64_t N, int d, int f, int E,
                                      const int32_t* offsets,
                                      const void* wg, const void* wv, const void* wo,
                                      const int64_t* rows, int64_t nrows, int x_compact,
                                      int store_bf16, const double* d_y, double* act,
                                      double* d_act, double* d_x)
{
    if (!x || !offsets || !wg || !wv || !wo || !rows || !d_y) return -1;
    if (d <= 0 || f <= 0 || E <= 0 || N < 0) return -1;
    if (offsets[0] != 0 || offsets[E] != N) return -2;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return -2;

#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)f);
        double* v = (double*)malloc(sizeof(double) * (size_t)f);
        double* dh = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t j = rows[r];
            int64_t xr = x_compact ? r : j;
            int e = expert_of(offsets, E, j);
            size_t wbase = (size_t)e * (size_t)d * (size_t)f;
            /* forward pre-activations, as in oracle_expert_ffn_rows */
            for (int c = 0; c < f; ++c) { a[c] = 0.0; v[c] = 0.0; }
            for (int i = 0; i < d; ++i) {
                double xi = (double)load_f(x, xtype, (size_t)xr * d + i);
                size_t wrow = wbase + (size_t)i * f;
                for (int c = 0; c < f; ++c) {
                    a[c] += xi * (double)load_f(wg, xtype, wrow + c);
                    v[c] += xi * (double)load_f(wv, xtype, wrow + c);
                }
            }
            /* y = h Wo  ->  dh_c = sum_o dy_o Wo[c,o] (dy as stored) */
            const double* dy = d_y + (size_t)r * d;
            const int rdy = store_bf16 & ORACLE_STORE_DY;
            for (int c = 0; c < f; ++c) {
                size_t wrow = wbase + (size_t)c * d;
                double acc = 0.0;
                for (int o = 0; o < d; ++o)
                    acc += (rdy ? round_bf16(dy[o]) : dy[o]) * (double)load_f(wo, xtype, wrow + o);
                dh[c] = acc;
            }
            if (store_bf16 & ORACLE_STORE_ACT)
                for (int c = 0; c < f; ++c) { a[c] = round_bf16(a[c]); v[c] = round_bf16(v[c]); }
            if (act)
                for (int c = 0; c < f; ++c) {
                    act[(size_t)r * 2 * f + c] = a[c];
                    act[(size_t)r * 2 * f + f + c] = v[c];
                }
            /* h = silu(a) v, silu(a) = a s, s = 1/(1+exp(-a)), silu'(a) = s (1 + a (1 - s)):
             * da = dh v silu'(a), dv = dh silu(a); stored over a and v */
            for (int c = 0; c < f; ++c) {
                double s = 1.0 / (1.0 + exp(-a[c]));
                double da = dh[c] * v[c] * (s * (1.0 + a[c] * (1.0 - s)));
                double dv = dh[c] * (a[c] * s);
                a[c] = (store_bf16 & ORACLE_STORE_DACT) ? round_bf16(da) : da;
                v[c] = (store_bf16 & ORACLE_STORE_DACT) ? round_bf16(dv) : dv;
            }
            if (d_act)
                for (int c = 0; c < f; ++c) {
                    d_act[(size_t)r * 2 * f + c] = a[c];
                    d_act[(size_t)r * 2 * f + f + c] = v[c];
                }
            /* a = x Wg, v = x Wv  ->  dx_i = sum_c da_c Wg[i,c] + dv_c Wv[i,c] */
            if (d_x)
                for (int i = 0; i < d; ++i) {
                    size_t wrow = wbase + (size_t)i * f;
                    double acc = 0.0;
                    for (int c = 0; c < f; ++c)
                        acc += a[c] * (double)load_f(wg, xtype, wrow + c)
                             + v[c] * (double)load_f(wv, xtype, wrow + c);
                    d_x[(size_t)r * d + i] = (store_bf16 & ORACLE_STORE_DX) ? round_bf16(acc) : acc;
                }
        }
        free(a);
        free(v);
        free(dh);
    }
    return 0;
}

int oracle_expert_weight_grads(const void* x, int xtype, int64_t N, int d, int f, int E,
                               const int32_t* offsets,
                               const void* wg, const void* wv, const void* wo,
                               const double* d_y, const int32_t* pair_e, const int32_t* pair_c,
                               int64_t npairs, double scale,
                               double* dwg, double* dwv, double* dwo)
{
    return oracle_expert_weight_grads_h(x, xtype, N, d, f, E, offsets, wg, wv, wo, d_y, pair_e,
                                        pair_c, npairs, scale, 0, dwg, dwv, dwo);
}

int oracle_expert_weight_grads_h(const void* x, int xtype, int64_t N, int d, int f, int E,
                                 const int32_t* offsets,
                                 const void* wg, const void* wv, const void* wo,
                                 const double* d_y, const int32_t* pair_e, const int32_t* pair_c,
                                 int64_t npairs, double scale, int store_bf16,
                                 double* dwg, double* dwv, double* dwo)
{
    if (!x || !offsets || !wg || !wv || !wo || !d_y || !pair_e || !pair_c) return -1;
    if (!dwg || !dwv || !dwo || d <= 0 || f <= 0 || E <= 0 || N < 0) return -1;
    if (offsets[0] != 0 || offsets[E] != N) return -2;
    for (int64_t p = 0; p < npairs; ++p)
        if (pair_e[p] < 0 || pair_e[p] >= E || pair_c[p] < 0 || pair_c[p] >= f) return -2;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < npairs; ++p) {
        int e = pair_e[p], c = pair_c[p];
        size_t wbase = (size_t)e * (size_t)d * (size_t)f;
        double* og = dwg + (size_t)p * d;
        double* ov = dwv + (size_t)p * d;
        double* oo = dwo + (size_t)p * d;
        for (int i = 0; i < d; ++i) { og[i] = 0.0; ov[i] = 0.0; oo[i] = 0.0; }
        for (int64_t j = offsets[e]; j < offsets[e + 1]; ++j) {
            /* column c of this row's pre-activations and of dh */
            double a = 0.0, v = 0.0, dh = 0.0;
            for (int i = 0; i < d; ++i) {
                double xi = (double)load_f(x, xtype, (size_t)j * d + i);
                a += xi * (double)load_f(wg, xtype, wbase + (size_t)i * f + c);
                v += xi * (double)load_f(wv, xtype, wbase + (size_t)i * f + c);
            }
            const double* dy = d_y + (size_t)j * d;
            const int rdy = store_bf16 & ORACLE_STORE_DY;
            for (int o = 0; o < d; ++o)
                dh += (rdy ? round_bf16(dy[o]) : dy[o]) * (double)load_f(wo, xtype, wbase + (size_t)c * d + o);
            /* h as the forward stored it (from the exact a and v) */
            double h = a * (1.0 / (1.0 + exp(-a))) * v;
            if (store_bf16 & ORACLE_STORE_ACT) {
                h = round_bf16(h);
                a = round_bf16(a);
                v = round_bf16(v);
            }
            double s = 1.0 / (1.0 + exp(-a));
            double da = dh * v * (s * (1.0 + a * (1.0 - s)));
            double dv = dh * (a * s);
            if (store_bf16 & ORACLE_STORE_DACT) { da = round_bf16(da); dv = round_bf16(dv); }
            /* a = x Wg[:,c]: dWg[i,c] += x_i da; likewise Wv; y = h Wo: dWo[c,o] += h dy_o */
            for (int i = 0; i < d; ++i) {
                double xi = (double)load_f(x, xtype, (size_t)j * d + i);
                og[i] += xi * da;
                ov[i] += xi * dv;
            }
            for (int o = 0; o < d; ++o) oo[o] += h * (rdy ? round_bf16(dy[o]) : dy[o]);
        }
        for (int i = 0; i < d; ++i) { og[i] *= scale; ov[i] *= scale; oo[i] *= scale; }
    }
    return 0;
}

/* ---------------------------------------------------- load statistics */

int oracle_route_stats(const float* logits, const int32_t* counts, int64_t T, int E, int k,
                       double* p_mean, double* aux)
{
    if (!logits || !counts || !p_mean || !aux || T <= 0 || E <= 0 || k <= 0) return -1;
    for (int e = 0; e < E; ++e) p_mean[e] = 0.0;
    /* full-softmax probability of every expert, averaged over the tokens */
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        double m = (double)l[0];
        for (int e = 1; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
        for (int e = 0; e < E; ++e) p_mean[e] += exp((double)l[e] - m) / z;
    }
    for (int e = 0; e < E; ++e) p_mean[e] /= (double)T;
    /* E * sum_e (share of the T*k assignments routed to e) * (mean probability of e) */
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += ((double)counts[e] / ((double)T * k)) * p_mean[e];
    *aux = (double)E * s;
    return 0;
}
