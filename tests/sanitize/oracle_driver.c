/*
 * Test driver: runs every oracle function once on seeded inputs (m = 8 and
 * m = 4, the Self-Indexing workload, attention and exact top-k), for a
 * build of oracle.c with the address and undefined-behaviour sanitizers.
 * Prints "ok" and exits 0 when every call returns 0; a sanitizer report
 * aborts the run.  Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_encode_keys(int d, int m, const int8_t *signs, int64_t n, const float *X,
                    uint8_t *ids, uint8_t *nib, uint16_t *w);
int orc_query_prep(int d, int m, int rho, const int32_t *tiers, const int8_t *signs, int G,
                   const float *Q, float *yq, uint8_t *lut, int32_t *top);
int orc_vote_scores(int B, int m, int64_t N, int64_t S, const uint8_t *ids,
                    const uint8_t *lut, int32_t *scores);
int64_t orc_cand_count(int64_t E, int64_t kprime, int64_t num, int64_t den);
int orc_candidates(int64_t E, int64_t S, const int32_t *scores, int64_t C, int32_t *cand);
int orc_rerank(int d, int m, const uint8_t *nib, const uint16_t *w, const float *yq,
               int64_t C, const int32_t *cand, float *est);
int orc_topk(int64_t C, const int32_t *cand, const float *est, int64_t kprime, int64_t S,
             int32_t *out);
int orc_attention(int d, int G, int64_t k, const float *Q, const float *K, const float *V,
                  const int32_t *idx, double scale, double *out);
int orc_exact_topk(int d, int G, const float *Q, int64_t N, int64_t S, const float *K,
                   int64_t kprime, int64_t *out);
int orc_si_build(int d, int64_t n, int64_t S, const float *X, float *mean, uint8_t *ids,
                 float *cb);
int orc_si_ids(int d, int64_t n, const float *X, const float *mean, uint8_t *ids);
int orc_si_lut(int d, int G, const float *Q, const float *cb, float *lut);
int orc_si_scores(int d, int64_t n, int64_t S, const uint8_t *ids, const float *lut,
                  float *scores);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static float rnd(void) {  /* xorshift64*, uniform in [-1, 1) */
    st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
    return (float)((st * 0x2545F4914F6CDD1Dull) >> 40) / (float)(1 << 23) - 1.0f;
}

#define CHECK(x) do { if ((x) != 0) { printf("failed: %s\n", #x); return 1; } } while (0)

int main(void) {
    enum { D = 128, N = 3000, S = 8, G = 4, K = 200 };
    float *X = malloc(sizeof(float) * N * D), *Q = malloc(sizeof(float) * G * D);
    float *V = malloc(sizeof(float) * N * D);
    int8_t signs[D];
    for (int i = 0; i < N * D; i++) { X[i] = rnd() * 3.0f; V[i] = rnd(); }
    for (int i = 0; i < G * D; i++) Q[i] = rnd();
    for (int j = 0; j < D; j++) signs[j] = rnd() < 0 ? -1 : 1;
    const int32_t tiers[4] = {4, 3, 2, 1};
    for (int m = 4; m <= 8; m += 4) {
        const int B = D / m, P = 1 << m;
        uint8_t *ids = malloc((size_t)N * B), *nib = malloc((size_t)N * D / 2);
        uint16_t *w = malloc(sizeof(uint16_t) * N * B);
        float yq[D];
        uint8_t *lut = malloc((size_t)B * P);
        int32_t *top = malloc(sizeof(int32_t) * B * 4);
        int32_t *sc = malloc(sizeof(int32_t) * N);
        CHECK(orc_encode_keys(D, m, signs, N, X, ids, nib, w));
        CHECK(orc_query_prep(D, m, 4, tiers, signs, G, Q, yq, lut, top));
        CHECK(orc_vote_scores(B, m, N, S, ids, lut, sc));
        const int64_t C = orc_cand_count(N - S, K - S, 1, 10);
        int32_t *cand = malloc(sizeof(int32_t) * C), out[K];
        float *est = malloc(sizeof(float) * C);
        CHECK(orc_candidates(N - S, S, sc, C, cand));
        CHECK(orc_rerank(D, m, nib, w, yq, C, cand, est));
        CHECK(orc_topk(C, cand, est, K - S, S, out));
        double *att = malloc(sizeof(double) * G * D);
        CHECK(orc_attention(D, G, K, Q, X, V, out, 0.088, att));
        free(ids); free(nib); free(w); free(lut); free(top); free(sc); free(cand); free(est);
        free(att);
    }
    int64_t ex[K - S];
    CHECK(orc_exact_topk(D, G, Q, N, S, X, K - S, ex));
    float mean[D], *cb = malloc(sizeof(float) * 32 * 16 * 4), lut[32 * 16];
    uint8_t *sids = malloc((size_t)N * 32);
    float *ssc = malloc(sizeof(float) * N);
    CHECK(orc_si_build(D, N - 100, S, X, mean, sids, cb));
    CHECK(orc_si_ids(D, 100, X + (size_t)(N - 100) * D, mean, sids + (size_t)(N - 100) * 32));
    CHECK(orc_si_lut(D, G, Q, cb, lut));
    CHECK(orc_si_scores(D, N, S, sids, lut, ssc));
    free(cb); free(sids); free(ssc); free(X); free(Q); free(V);
    printf("ok\n");
    return 0;
}
