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

int oracle_expert_ffn_rows(const void* x, int xtype, int64_t N, int d, int f, int E,
                           const int32_t* offsets,
                           const void* wg, const void* wv, const void* wo,
                           const int64_t* rows, int64_t nrows, int x_compact, double* y)
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
