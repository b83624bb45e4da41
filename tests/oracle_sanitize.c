/*
 * Driver for the sanitizer run of the oracle (tests/test_oracle_sanitize.py):
 * compiled together with oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (no OpenMP), it calls every oracle entry point
 * on small seeded inputs, edge cases included (empty experts, k = E, one
 * expert taking every token, capacity 0, dropped ids, fp32 and bf16 data),
 * so that an out-of-bounds access, a leak or undefined behaviour anywhere
 * in the oracle aborts the run. Returns 0 when every call succeeded (or
 * failed exactly where the input breaks a stated precondition).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.h"

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* splitmix64 */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

/* uniform in [-1, 1) */
static float uni(void) { return (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0); }

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void* fill(size_t n, int xtype, float scale) {
    if (xtype == 0) {
        float* p = malloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) p[i] = uni() * scale;
        return p;
    }
    uint16_t* p = malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) p[i] = to_bf16(uni() * scale);
    return p;
}

static int failures = 0;
#define EXPECT(call, want)                                                        \
    do {                                                                          \
        int rc_ = (call);                                                         \
        if (rc_ != (want)) {                                                      \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__,     \
                    __LINE__, #call, rc_, (want));                                \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static void layer(int xtype, int T, int d, int f, int E, int k, int renorm, float bias_hot) {
    const int64_t TK = (int64_t)T * k;
    void* x = fill((size_t)T * d, xtype, 1.0f);
    void* w = fill((size_t)d * E, xtype, 0.05f);
    void* wg = fill((size_t)E * d * f, xtype, 0.1f);
    void* wv = fill((size_t)E * d * f, xtype, 0.1f);
    void* wo = fill((size_t)E * f * d, xtype, 0.1f);
    float* bias = malloc(E * sizeof(float));
    for (int e = 0; e < E; ++e) bias[e] = 0.5f * uni();
    if (bias_hot != 0.0f) bias[E - 1] = bias_hot;   /* one expert takes every token */
    if (E > 4) bias[1] = -1.0e4f;                    /* an expert that gets nothing */

    float* logits = malloc((size_t)T * E * sizeof(float));
    int32_t* idx = malloc(TK * sizeof(int32_t));
    double* gates = malloc(TK * sizeof(double));
    EXPECT(oracle_route(x, w, xtype, bias, T, d, E, k, renorm, logits, idx, gates), 0);

    int32_t* counts = malloc(E * sizeof(int32_t));
    int32_t* routed = malloc(E * sizeof(int32_t));
    int32_t* offsets = malloc((E + 1) * sizeof(int32_t));
    int32_t* perm_src = malloc((TK + 1) * sizeof(int32_t));
    int32_t* dest = malloc((TK + 1) * sizeof(int32_t));
    EXPECT(oracle_permute(idx, TK, E, counts, offsets, perm_src, dest), 0);
    EXPECT(oracle_permute_capacity(idx, TK, E, 0, routed, counts, offsets, perm_src, dest), 0);
    EXPECT(oracle_permute_capacity(idx, TK, E, 3, routed, counts, offsets, perm_src, dest), 0);
    EXPECT(oracle_permute_capacity(idx, TK, E, -1, routed, counts, offsets, perm_src, dest), -1);
    EXPECT(oracle_permute_range(idx, TK, E / 2, E - E / 2, counts, offsets, perm_src, dest), 0);
    EXPECT(oracle_permute(idx, TK, E, counts, offsets, perm_src, dest), 0);

    const int es = xtype ? 2 : 4;
    void* xp = malloc((size_t)TK * d * es);
    EXPECT(oracle_gather(x, es, d, perm_src, TK, k, xp), 0);
    int64_t* rows = malloc(TK * sizeof(int64_t));
    for (int64_t j = 0; j < TK; ++j) rows[j] = j;
    double* y = malloc((size_t)TK * d * sizeof(double));
    EXPECT(oracle_expert_ffn_rows(xp, xtype, TK, d, f, E, offsets, wg, wv, wo, rows, TK, 0, y), 0);
    int32_t* tokens = malloc(T * sizeof(int32_t));
    for (int t = 0; t < T; ++t) tokens[t] = t;
    double* out = malloc((size_t)T * d * sizeof(double));
    EXPECT(oracle_combine(tokens, T, k, d, dest, gates, y, NULL, NULL, out), 0);
    EXPECT(oracle_combine(tokens, T, k, d, dest, NULL, y, NULL, out, out), 0);

    /* backward */
    double* dout = malloc((size_t)T * d * sizeof(double));
    for (size_t i = 0; i < (size_t)T * d; ++i) dout[i] = uni();
    double* dg = malloc(TK * sizeof(double));
    EXPECT(oracle_combine_backward_gates(tokens, T, k, d, dest, y, NULL, dout, dg), 0);
    double* dy = malloc((size_t)TK * d * sizeof(double));
    EXPECT(oracle_combine_backward_rows(perm_src, rows, TK, k, d, gates, dout, dy), 0);
    double* act = malloc((size_t)TK * 2 * f * sizeof(double));
    double* dact = malloc((size_t)TK * 2 * f * sizeof(double));
    double* dxp = malloc((size_t)TK * d * sizeof(double));
    EXPECT(oracle_expert_ffn_backward_rows(xp, xtype, TK, d, f, E, offsets, wg, wv, wo, rows, TK,
                                           0, dy, act, dact, dxp), 0);
    int32_t pe[3] = {0, E - 1, E / 2}, pc[3] = {0, f - 1, f / 2};
    double* dwg = malloc(3 * (size_t)d * sizeof(double));
    double* dwv = malloc(3 * (size_t)d * sizeof(double));
    double* dwo = malloc(3 * (size_t)d * sizeof(double));
    EXPECT(oracle_expert_weight_grads(xp, xtype, TK, d, f, E, offsets, wg, wv, wo, dy, pe, pc, 3,
                                      0.25, dwg, dwv, dwo), 0);
    /* the storage-point variants (bf16 rounding where training stores values) */
    EXPECT(oracle_expert_ffn_rows_h(xp, xtype, TK, d, f, E, offsets, wg, wv, wo, rows, TK, 0, 1, y), 0);
    EXPECT(oracle_expert_ffn_backward_rows_h(xp, xtype, TK, d, f, E, offsets, wg, wv, wo, rows, TK,
                                             0, 15, dy, act, dact, dxp), 0);
    EXPECT(oracle_expert_weight_grads_h(xp, xtype, TK, d, f, E, offsets, wg, wv, wo, dy, pe, pc, 3,
                                        0.25, 7, dwg, dwv, dwo), 0);
    EXPECT(oracle_round_bf16(dy, (int64_t)TK * d), 0);
    double* dl = malloc((size_t)T * E * sizeof(double));
    EXPECT(oracle_route_backward(logits, idx, gates, dg, T, E, k, renorm, dl), 0);
    double* dx = malloc((size_t)T * d * sizeof(double));
    double* dw = malloc((size_t)d * E * sizeof(double));
    EXPECT(oracle_router_grads(x, w, xtype, T, d, E, dl, tokens, T, dx, dw), 0);
    double pm[64], aux;
    if (E <= 64) {
        EXPECT(oracle_permute(idx, TK, E, counts, offsets, perm_src, dest), 0);
        EXPECT(oracle_route_stats(logits, counts, T, E, k, pm, &aux), 0);
    }
    /* an id outside [0,E) breaks the packing's precondition */
    idx[TK - 1] = E;
    EXPECT(oracle_permute(idx, TK, E, counts, offsets, perm_src, dest), -2);

    free(x); free(w); free(wg); free(wv); free(wo); free(bias); free(logits); free(idx);
    free(gates); free(counts); free(routed); free(offsets); free(perm_src); free(dest); free(xp);
    free(rows); free(y); free(tokens); free(out); free(dout); free(dg); free(dy); free(act);
    free(dact); free(dxp); free(dwg); free(dwv); free(dwo); free(dl); free(dx); free(dw);
}

static void receive(void) {
    const int S = 3, E = 5;
    int32_t recv[15];
    int64_t N = 0;
    for (int c = 0; c < S * E; ++c) {
        recv[c] = (c % 4 == 0) ? 0 : (int32_t)(next_u64() % 7);
        N += recv[c];
    }
    int32_t counts[5], offsets[6];
    int32_t* perm_src = malloc((N + 1) * sizeof(int32_t));
    int32_t* dest = malloc((N + 1) * sizeof(int32_t));
    EXPECT(oracle_permute_recv(recv, S, E, N, counts, offsets, perm_src, dest), 0);
    EXPECT(oracle_permute_recv(recv, S, E, N + 1, counts, offsets, perm_src, dest), -2);
    free(perm_src);
    free(dest);
}

int main(void) {
    layer(0, 37, 48, 80, 5, 3, 1, 0.0f);     /* fp32, odd sizes */
    layer(1, 64, 32, 16, 8, 2, 0, 0.0f);     /* bf16, full-softmax weights */
    layer(1, 20, 16, 16, 6, 6, 1, 0.0f);     /* k = E */
    layer(0, 9, 8, 8, 4, 1, 1, 1.0e4f);      /* one expert takes every token, k = 1 */
    receive();
    if (failures) {
        fprintf(stderr, "%d oracle call(s) returned an unexpected code\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: every call ok\n");
    return 0;
}
