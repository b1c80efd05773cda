/*
 * CPU oracle for the ParisKV per-decode-step KV-cache retrieval path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; it derives its own rotation, codebook,
 * fp16 rounding and sorting from the method's definition.
 *
 * Sources (cited by page title and section):
 *   [TS]  "Technical Summary: ParisKV" (gist.science/paper/2602.07721)
 *         - Core Algorithmic Innovations 1 "Drift-Robust Analytic Centroids":
 *           l2 normalisation + shared random orthogonal rotation (SRHT);
 *           analytic sign-pattern centroids (+-1/sqrt(m)).
 *         - Core Algorithmic Innovations 2 "Two-Stage GPU-Native Retrieval
 *           Pipeline": Coarse Candidate Generation (B subspaces, nearest
 *           centroid, top-rho query centroids, tiered votes, top fraction)
 *           and Candidate Reranking (RSQ-IP: 4-bit code = 1 sign bit +
 *           3 magnitude bits from the rotation-induced Beta prior; calibration
 *           w_{i,b}; estimator ||q|| sum_b w_{i,b} <v_{i,b}, q~_b>).
 *         - Problem Statement: sparse attention over the Top-k past tokens.
 *   [ICML] "ParisKV: Fast and Drift-Robust KV-Cache Retrieval for
 *          Long-Context LLMs" (ICML 2026 poster abstract): collision-based
 *          candidate selection followed by quantised inner-product reranking.
 *   [SI]  "Self-Indexing KVCache: Predicting Sparse Attention from
 *         Compressed Keys" (gist.science/paper/2603.14224), Methodology A-C:
 *         the second workload (channel-mean centring, 4-dim sign-pattern
 *         clusters with mean centroids, LUT-GEMV scores, sink tokens).
 *
 * Where the pages leave a step open, the plainest reading is taken; each
 * such reading is stated at the function that implements it.
 *
 * Floating point: compiled with -O2 -ffp-contract=off, no fast-math.  Every
 * step that decides an integer (bucket ids, codes, centroid ranking) runs in
 * fp32 in a fixed, stated order, because the kernel under test decides those
 * integers in fp32 too.  Attention and the exact inner-product reference run
 * in fp64.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* ------------------------------------------------------------------------ */
/* fp16 round-to-nearest-even (own implementation of IEEE 754 binary16).     */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits = f32_bits(f);
    uint16_t s = (uint16_t)((bits >> 16) & 0x8000u);
    uint32_t x = bits & 0x7FFFFFFFu;
    if (x >= 0x7F800000u)                      /* inf or NaN */
        return (uint16_t)(s | (x > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (x >= 0x477FF000u)                      /* >= 65520 rounds to inf */
        return (uint16_t)(s | 0x7C00u);
    if (x >= 0x38800000u) {                    /* >= 2^-14: normal half */
        uint32_t e = (x >> 23) - 127u + 15u;
        uint32_t m = x & 0x7FFFFFu;
        uint32_t h = (e << 10) | (m >> 13);
        uint32_t rem = m & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))
            h++;                               /* carry may bump exponent */
        return (uint16_t)(s | h);
    }
    /* half subnormal range: value / 2^-24 rounded to an integer, RNE */
    {
        uint32_t e = x >> 23;
        if (e < 102u)                          /* < 2^-25 (or float subnormal) */
            return s;
        uint32_t m = (x & 0x7FFFFFu) | 0x800000u;  /* value = m * 2^(e-150) */
        uint32_t shift = 126u - e;                 /* 14 .. 24 */
        uint32_t h = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1u);
        if (rem > half || (rem == half && (h & 1u)))
            h++;
        return (uint16_t)(s | h);
    }
}

float orc_f16_to_f32(uint16_t h)
{
    uint32_t s = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t m = (uint32_t)h & 0x3FFu;
    if (e == 0x1Fu)
        return bits_f32(s | 0x7F800000u | (m << 13));
    if (e == 0) {
        /* zero or subnormal: exact value m * 2^-24 */
        float v = (float)m * 5.9604644775390625e-08f; /* 2^-24, exact */
        return s ? -v : v;
    }
    return bits_f32(s | ((e - 15u + 127u) << 23) | (m << 13));
}

/* ------------------------------------------------------------------------ */
/* RSQ-IP magnitude codebook.                                               */
/*                                                                          */
/* [TS] RSQ-IP "Quantization": each subspace direction gets 1 sign bit and  */
/* 3 magnitude bits derived from the rotation-induced Beta prior.           */
/* Reading: the code is per coordinate of the unit subspace direction u     */
/* (m coordinates, 4 bits each).  After a random rotation u is uniform on   */
/* the unit sphere S^{m-1}, so u_j^2 ~ Beta(1/2, (m-1)/2) and t = |u_j| has */
/* density proportional to (1 - t^2)^((m-3)/2) on [0, 1].  The 8 magnitude  */
/* levels are the Lloyd-Max (minimum mean squared error) scalar quantiser   */
/* of t under that density: thresholds are midpoints of adjacent levels and */
/* each level is the conditional mean of its cell.                          */
/*                                                                          */
/* Computed here in double with the substitution t = sin(theta), which      */
/* turns both cell integrals into smooth integrals of cos^(m-2)(theta) and  */
/* sin(theta) cos^(m-2)(theta), evaluated by composite Simpson's rule, and  */
/* the Lloyd iteration run to a fixed point.                                */
/* ------------------------------------------------------------------------ */

#define ORC_LEVELS 8
#define ORC_SIMPSON_N 512  /* even number of Simpson intervals per cell */

static void cell_moments(int m, double a, double b, double *mass, double *first)
{
    double ta = asin(a), tb = asin(b);
    double hstep = (tb - ta) / ORC_SIMPSON_N;
    double s0 = 0.0, s1 = 0.0;
    for (int i = 0; i <= ORC_SIMPSON_N; i++) {
        double th = ta + hstep * i;
        double c = cos(th);
        if (c < 0.0) c = 0.0;
        double g = (m == 2) ? 1.0 : pow(c, (double)(m - 2));
        double wgt = (i == 0 || i == ORC_SIMPSON_N) ? 1.0 : ((i & 1) ? 4.0 : 2.0);
        s0 += wgt * g;
        s1 += wgt * g * sin(th);
    }
    *mass = s0 * hstep / 3.0;
    *first = s1 * hstep / 3.0;
}

static int cb_ready[9];
static double cb_L[9][ORC_LEVELS];
static double cb_tau[9][ORC_LEVELS - 1];

int orc_codebook(int m, double *L, double *tau)
{
    if (m < 2 || m > 8)
        return ORC_EINVAL;
    if (!cb_ready[m]) {
        double lv[ORC_LEVELS], th[ORC_LEVELS + 1];
        for (int l = 0; l < ORC_LEVELS; l++)
            lv[l] = (l + 0.5) / ORC_LEVELS;
        th[0] = 0.0;
        th[ORC_LEVELS] = 1.0;
        for (int it = 0; it < 200000; it++) {
            for (int l = 1; l < ORC_LEVELS; l++)
                th[l] = 0.5 * (lv[l - 1] + lv[l]);
            double change = 0.0;
            for (int l = 0; l < ORC_LEVELS; l++) {
                double mass, first;
                cell_moments(m, th[l], th[l + 1], &mass, &first);
                double nl = first / mass;
                double dd = fabs(nl - lv[l]);
                if (dd > change) change = dd;
                lv[l] = nl;
            }
            if (change < 1e-16)
                break;
        }
        for (int l = 1; l < ORC_LEVELS; l++)
            th[l] = 0.5 * (lv[l - 1] + lv[l]);
        for (int l = 0; l < ORC_LEVELS; l++)
            cb_L[m][l] = lv[l];
        for (int l = 0; l < ORC_LEVELS - 1; l++)
            cb_tau[m][l] = th[l + 1];
        cb_ready[m] = 1;
    }
    if (L) memcpy(L, cb_L[m], sizeof(double) * ORC_LEVELS);
    if (tau) memcpy(tau, cb_tau[m], sizeof(double) * (ORC_LEVELS - 1));
    return ORC_OK;
}

/* fp32 copies used by the encoder and the estimator (nearest fp32). */
int orc_codebook_f32(int m, float *L32, float *tau32)
{
    double L[ORC_LEVELS], tau[ORC_LEVELS - 1];
    int rc = orc_codebook(m, L, tau);
    if (rc) return rc;
    for (int l = 0; l < ORC_LEVELS; l++) L32[l] = (float)L[l];
    for (int l = 0; l < ORC_LEVELS - 1; l++) tau32[l] = (float)tau[l];
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Shared random orthogonal rotation (SRHT).                                */
/*                                                                          */
/* [TS] Core 1 "Normalization and Rotation": keys and queries get the same  */
/* random orthogonal rotation, implemented via SRHT.                        */
/* Reading: one round R = c * H * diag(D), H the Sylvester-ordered d x d    */
/* Hadamard matrix, D random signs (an input), c = fp32 nearest 1/sqrt(d),  */
/* no row subsampling (an orthogonal map is square).  Evaluated in fp32:    */
/* sign flip, then the butterfly stages h = 1, 2, 4, ..., d/2 in that order */
/* with (a, b) -> (a + b, a - b) for the pair (j, j + h), then * c.          */
/* ------------------------------------------------------------------------ */

/* The diagonal D from a seed: D_j = -1 when bit 63 of the j-th output    */
/* (j = 0 .. d-1) of SplitMix64 seeded with `seed` is set, else +1.       */
/* SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom       */
/* Number Generators", OOPSLA 2014): the state advances by the odd        */
/* constant 0x9e3779b97f4a7c15; each output is the state passed through   */
/* two xor-shift-multiply rounds (shifts 30 and 27, multipliers            */
/* 0xbf58476d1ce4e5b9 and 0x94d049bb133111eb) and a final xor-shift by 31. */
int orc_srht_signs(uint64_t seed, int d, int8_t *D)
{
    if (d < 1) return ORC_EINVAL;
    uint64_t state = seed;
    for (int j = 0; j < d; j++) {
        state += 0x9e3779b97f4a7c15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        z = z ^ (z >> 31);
        D[j] = (z >> 63) ? -1 : 1;
    }
    return ORC_OK;
}

/* Raw SplitMix64 outputs (the generator's known-answer pin). */
int orc_splitmix64(uint64_t seed, int n, uint64_t *out)
{
    if (n < 0) return ORC_EINVAL;
    uint64_t state = seed;
    for (int j = 0; j < n; j++) {
        state += 0x9e3779b97f4a7c15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        out[j] = z ^ (z >> 31);
    }
    return ORC_OK;
}

float orc_rot_scale(int d)
{
    return (float)(1.0 / sqrt((double)d));
}

int orc_rotate(int d, const int8_t *signs, const float *x, float *y)
{
    if (d < 2 || (d & (d - 1)))
        return ORC_EINVAL;
    for (int j = 0; j < d; j++)
        y[j] = (signs[j] < 0) ? -x[j] : x[j];
    for (int h = 1; h < d; h <<= 1)
        for (int blk = 0; blk < d; blk += 2 * h)
            for (int j = blk; j < blk + h; j++) {
                float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    float c = orc_rot_scale(d);
    for (int j = 0; j < d; j++)
        y[j] = y[j] * c;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Key encoding (index build and incremental append).                        */
/*                                                                          */
/* [TS] Coarse Candidate Generation: the rotated key is split into B        */
/* subspaces and each subspace direction is assigned to the nearest         */
/* analytic centroid.  Reading: contiguous blocks of m = d/B coordinates;   */
/* centroid p has coordinate j equal to -1/sqrt(m) if bit j of p is set,   */
/* else +1/sqrt(m); the nearest centroid of z is its sign pattern, so the   */
/* bucket id is sum_j [z_j < 0] 2^j (a zero goes to the + side).  The       */
/* normalisation of the key is folded into the calibration factor: signs   */
/* and directions do not depend on the scale.                               */
/*                                                                          */
/* [TS] Candidate Reranking (RSQ-IP) Quantization + Calibration:            */
/*   n  = ||z|| (fp32: sequential sum of z_j*z_j, correctly rounded sqrt)   */
/*   u  = z / n                                                             */
/*   code_j = (sign_j << 3) | mag_j, mag_j = #{l : |u_j| >= tau_l}          */
/*   v_j = (sign_j ? -1 : +1) * L[mag_j]   (the dequantised direction)      */
/*   w = fp16(n / <v, u>)                                                   */
/* Reading of w: the alignment-corrected factor, so that w <v, q_b> is the  */
/* unbiased inner-product estimate n <u, q_b> when the quantisation error   */
/* is orthogonal to q_b, and is exact for q_b parallel to u.  It carries    */
/* the subspace norm, i.e. the key's l2 norm.  A zero subspace gets all     */
/* magnitudes 0 and w = 0.                                                   */
/* Packing: coordinate j of the key is nibble j; byte j/2 holds coordinate  */
/* 2p in its low nibble and 2p+1 in its high nibble.                        */
/* ------------------------------------------------------------------------ */

int orc_encode_keys(int d, int m, const int8_t *signs, int64_t n,
                    const float *X, uint8_t *ids, uint8_t *nib, uint16_t *w)
{
    if (d < 2 || (d & (d - 1)) || m < 2 || m > 8 || d % m)
        return ORC_EINVAL;
    int B = d / m;
    float L32[ORC_LEVELS], tau32[ORC_LEVELS - 1];
    if (orc_codebook_f32(m, L32, tau32))
        return ORC_EINVAL;
    float *y = (float *)malloc(sizeof(float) * d);
    if (!y) return ORC_EINVAL;
    for (int64_t i = 0; i < n; i++) {
        orc_rotate(d, signs, X + i * d, y);
        uint8_t *kid = ids + i * B;
        uint8_t *knib = nib + i * (d / 2);
        uint16_t *kw = w + i * B;
        memset(knib, 0, (size_t)(d / 2));
        for (int b = 0; b < B; b++) {
            const float *z = y + b * m;
            unsigned id = 0;
            for (int j = 0; j < m; j++)
                if (z[j] < 0.0f)
                    id |= 1u << j;
            kid[b] = (uint8_t)id;

            float n2 = 0.0f;
            for (int j = 0; j < m; j++)
                n2 = n2 + z[j] * z[j];
            float nrm = sqrtf(n2);

            unsigned code[8];
            float a = 0.0f;
            for (int j = 0; j < m; j++) {
                unsigned sgn = (id >> j) & 1u;
                unsigned mag = 0;
                float u = 0.0f;
                if (nrm != 0.0f) {
                    u = z[j] / nrm;
                    float au = fabsf(u);
                    for (int l = 0; l < ORC_LEVELS - 1; l++)
                        if (au >= tau32[l])
                            mag++;
                }
                code[j] = (sgn << 3) | mag;
                if (nrm != 0.0f) {
                    float v = sgn ? -L32[mag] : L32[mag];
                    a = a + v * u;
                }
            }
            kw[b] = (nrm != 0.0f) ? orc_f32_to_f16(nrm / a) : (uint16_t)0;
            for (int j = 0; j < m; j++) {
                int c = b * m + j;
                knib[c >> 1] |= (uint8_t)(code[j] << ((c & 1) ? 4 : 0));
            }
        }
    }
    free(y);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Query preparation.                                                       */
/*                                                                          */
/* Reading for grouped-query attention: one retrieval per (batch, KV head); */
/* its query is the mean of the G query heads that share the KV head (fp32: */
/* q_0 + q_1 + ... in head order, then * fp32(1/G)).  Its exact top-k is    */
/* the top-k of the group-summed logits.                                    */
/* [TS] Coarse Candidate Generation: per subspace, the query selects the    */
/* rho centroids most similar to its rotated sub-vector; keys in those      */
/* buckets get tiered votes.  Reading: similarity is the inner product with */
/* the centroid (all centroids have one norm, so this is the cosine); the   */
/* score of centroid p is, in fp32, the sum over j in order of (bit j of p  */
/* ? -yq_j : +yq_j) (the 1/sqrt(m) factor does not change the order); rank  */
/* by (score descending, p ascending); the s-th ranked centroid gets        */
/* weight tiers[s-1], every other centroid 0.                               */
/* ------------------------------------------------------------------------ */

int orc_query_prep(int d, int m, int rho, const int32_t *tiers,
                   const int8_t *signs, int G, const float *Q,
                   float *yq, uint8_t *lut, int32_t *top)
{
    if (d < 2 || (d & (d - 1)) || m < 2 || m > 8 || d % m || G < 1)
        return ORC_EINVAL;
    int B = d / m, P = 1 << m;
    if (rho < 1 || rho > P)
        return ORC_EINVAL;
    float *qb = (float *)malloc(sizeof(float) * d);
    float *sc = (float *)malloc(sizeof(float) * P);
    unsigned char *taken = (unsigned char *)malloc((size_t)P);
    if (!qb || !sc || !taken) { free(qb); free(sc); free(taken); return ORC_EINVAL; }
    float invG = 1.0f / (float)G;
    for (int j = 0; j < d; j++) {
        float acc = Q[j];
        for (int g = 1; g < G; g++)
            acc = acc + Q[(int64_t)g * d + j];
        qb[j] = acc * invG;
    }
    orc_rotate(d, signs, qb, yq);
    for (int b = 0; b < B; b++) {
        const float *z = yq + b * m;
        for (int p = 0; p < P; p++) {
            float s = (p & 1) ? -z[0] : z[0];
            for (int j = 1; j < m; j++)
                s = s + (((p >> j) & 1) ? -z[j] : z[j]);
            sc[p] = s;
        }
        memset(taken, 0, (size_t)P);
        uint8_t *lb = lut + (int64_t)b * P;
        memset(lb, 0, (size_t)P);
        for (int r = 0; r < rho; r++) {
            int best = -1;
            for (int p = 0; p < P; p++) {
                if (taken[p]) continue;
                if (best < 0 || sc[p] > sc[best])
                    best = p;               /* strict >: lower p wins ties */
            }
            taken[best] = 1;
            lb[best] = (uint8_t)tiers[r];
            if (top) top[b * rho + r] = best;
        }
    }
    free(qb); free(sc); free(taken);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Collision votes.                                                         */
/* [TS] Coarse Candidate Generation: votes are summed across subspaces into */
/* an integer coarse score.  score_i = sum_b lut_b[id_{i,b}], for keys      */
/* i in [S, N) (the S sink tokens are always selected and never scored).    */
/* ------------------------------------------------------------------------ */

int orc_vote_scores(int B, int m, int64_t N, int64_t S, const uint8_t *ids,
                    const uint8_t *lut, int32_t *scores)
{
    int P = 1 << m;
    for (int64_t i = S; i < N; i++) {
        int32_t s = 0;
        for (int b = 0; b < B; b++)
            s += lut[(int64_t)b * P + ids[i * B + b]];
        scores[i - S] = s;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Candidate set.                                                           */
/* [TS] Coarse Candidate Generation prunes to the top fraction (5-10%) of   */
/* keys by coarse score.  Reading: C = min(E, max(k', ceil(E f))) with f an */
/* exact rational, E = N - S, k' = k - S; the candidates are the first C    */
/* eligible keys in (score descending, index ascending) order, listed in    */
/* ascending index order.                                                    */
/* ------------------------------------------------------------------------ */

int64_t orc_cand_count(int64_t E, int64_t kprime, int64_t num, int64_t den)
{
    int64_t c = (E * num + den - 1) / den;
    if (c < kprime) c = kprime;
    if (c > E) c = E;
    return c;
}

typedef struct { int32_t key; int64_t idx; } orc_si;

static int cmp_score_desc_idx_asc(const void *pa, const void *pb)
{
    const orc_si *a = (const orc_si *)pa, *b = (const orc_si *)pb;
    if (a->key != b->key) return (a->key > b->key) ? -1 : 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

static int cmp_i64(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    return (a < b) ? -1 : (a > b);
}

static int cmp_i32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a < b) ? -1 : (a > b);
}

int orc_candidates(int64_t E, int64_t S, const int32_t *scores, int64_t C,
                   int32_t *cand)
{
    if (C < 0 || C > E)
        return ORC_EINVAL;
    orc_si *v = (orc_si *)malloc(sizeof(orc_si) * (size_t)(E > 0 ? E : 1));
    if (!v) return ORC_EINVAL;
    for (int64_t p = 0; p < E; p++) { v[p].key = scores[p]; v[p].idx = S + p; }
    qsort(v, (size_t)E, sizeof(orc_si), cmp_score_desc_idx_asc);
    for (int64_t c = 0; c < C; c++)
        cand[c] = (int32_t)v[c].idx;
    qsort(cand, (size_t)C, sizeof(int32_t), cmp_i32);
    free(v);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* RSQ-IP rerank.                                                           */
/* [TS] Candidate Reranking "Estimation": <k, q> ~ ||q|| sum_b w_{i,b}      */
/* <v_{i,b}, q~_b>, with v the dequantised direction and q~ the rotated     */
/* query.  Reading: ||q|| q~_b is the b-th block of yq = R q (the rotation  */
/* of the unnormalised group query, kept in fp32).  Order, in fp32 with no  */
/* fused multiply-add: est = 0; for b ascending { p = 0; for j ascending    */
/* p = p + v_{b,j} * yq_{b,j}; est = est + w_b * p }.                       */
/* ------------------------------------------------------------------------ */

int orc_rerank(int d, int m, const uint8_t *nib, const uint16_t *w,
               const float *yq, int64_t C, const int32_t *cand, float *est)
{
    if (d % m || m < 2 || m > 8) return ORC_EINVAL;
    int B = d / m;
    float L32[ORC_LEVELS], tau32[ORC_LEVELS - 1];
    if (orc_codebook_f32(m, L32, tau32)) return ORC_EINVAL;
    for (int64_t c = 0; c < C; c++) {
        int64_t i = cand[c];
        const uint8_t *kn = nib + i * (d / 2);
        const uint16_t *kw = w + i * B;
        float e = 0.0f;
        for (int b = 0; b < B; b++) {
            float p = 0.0f;
            for (int j = 0; j < m; j++) {
                int cc = b * m + j;
                unsigned code = (kn[cc >> 1] >> ((cc & 1) ? 4 : 0)) & 0xFu;
                float v = (code & 8u) ? -L32[code & 7u] : L32[code & 7u];
                p = p + v * yq[cc];
            }
            e = e + orc_f16_to_f32(kw[b]) * p;
        }
        est[c] = e;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Exact top-k over the reranked candidates.                                */
/* [TS] Key Contributions 2: high-fidelity Top-k selection on the           */
/* compressed codes.  Order (est descending, index ascending), -0 equal to  */
/* +0; take k' = k - S; the S sinks [0, S) are always in the selection.     */
/* Output ascending.                                                        */
/* ------------------------------------------------------------------------ */

typedef struct { float est; int32_t idx; } orc_ei;

static int cmp_est_desc_idx_asc(const void *pa, const void *pb)
{
    const orc_ei *a = (const orc_ei *)pa, *b = (const orc_ei *)pb;
    if (a->est > b->est) return -1;    /* float compare: -0 == +0 */
    if (a->est < b->est) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

int orc_topk(int64_t C, const int32_t *cand, const float *est, int64_t kprime,
             int64_t S, int32_t *out)
{
    if (kprime < 0 || kprime > C) return ORC_EINVAL;
    orc_ei *v = (orc_ei *)malloc(sizeof(orc_ei) * (size_t)(C > 0 ? C : 1));
    if (!v) return ORC_EINVAL;
    for (int64_t c = 0; c < C; c++) { v[c].est = est[c]; v[c].idx = cand[c]; }
    qsort(v, (size_t)C, sizeof(orc_ei), cmp_est_desc_idx_asc);
    for (int64_t s = 0; s < S; s++) out[s] = (int32_t)s;
    for (int64_t c = 0; c < kprime; c++) out[S + c] = v[c].idx;
    qsort(out, (size_t)(S + kprime), sizeof(int32_t), cmp_i32);
    free(v);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Sparse attention over the selected full-precision rows.                  */
/* [TS] Problem Statement: attend only to a Top-k subset of past tokens;    */
/* System-Level Innovations 1: only the selected Top-k K/V pairs are        */
/* fetched.  Reading: standard softmax attention with the caller's scale    */
/* (normally 1/sqrt(d)) over exactly the selected rows, per query head of   */
/* the group; computed in fp64 with a textbook max-shifted softmax.         */
/* K, V are row-major [rows][d] of fp32 values; idx selects rows.           */
/* ------------------------------------------------------------------------ */

int orc_attention(int d, int G, int64_t k, const float *Q, const float *K,
                  const float *V, const int32_t *idx, double scale, double *out)
{
    double *lg = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    if (!lg) return ORC_EINVAL;
    for (int g = 0; g < G; g++) {
        const float *q = Q + (int64_t)g * d;
        double mx = -INFINITY;
        for (int64_t t = 0; t < k; t++) {
            const float *kr = K + (int64_t)idx[t] * d;
            double s = 0.0;
            for (int j = 0; j < d; j++)
                s += (double)q[j] * (double)kr[j];
            lg[t] = s * scale;
            if (lg[t] > mx) mx = lg[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < k; t++) {
            lg[t] = exp(lg[t] - mx);
            den += lg[t];
        }
        double *o = out + (int64_t)g * d;
        for (int j = 0; j < d; j++) o[j] = 0.0;
        for (int64_t t = 0; t < k; t++) {
            const float *vr = V + (int64_t)idx[t] * d;
            double p = lg[t] / den;
            for (int j = 0; j < d; j++)
                o[j] += p * (double)vr[j];
        }
    }
    free(lg);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Exact inner-product top-k (the recall reference).                        */
/* The set the retrieval approximates: top k' keys in [S, N) by             */
/* <mean of the G query heads, k_i> in fp64, ties to the lower index.       */
/* ------------------------------------------------------------------------ */

typedef struct { double v; int64_t idx; } orc_di;

static int cmp_dv_desc_idx_asc(const void *pa, const void *pb)
{
    const orc_di *a = (const orc_di *)pa, *b = (const orc_di *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

int orc_exact_topk(int d, int G, const float *Q, int64_t N, int64_t S,
                   const float *K, int64_t kprime, int64_t *out)
{
    int64_t E = N - S;
    if (E < 0 || kprime > E) return ORC_EINVAL;
    double *qb = (double *)malloc(sizeof(double) * d);
    orc_di *v = (orc_di *)malloc(sizeof(orc_di) * (size_t)(E > 0 ? E : 1));
    if (!qb || !v) { free(qb); free(v); return ORC_EINVAL; }
    for (int j = 0; j < d; j++) {
        double a = 0.0;
        for (int g = 0; g < G; g++) a += (double)Q[(int64_t)g * d + j];
        qb[j] = a / G;
    }
    for (int64_t i = S; i < N; i++) {
        double s = 0.0;
        for (int j = 0; j < d; j++) s += qb[j] * (double)K[i * d + j];
        v[i - S].v = s;
        v[i - S].idx = i;
    }
    qsort(v, (size_t)E, sizeof(orc_di), cmp_dv_desc_idx_asc);
    for (int64_t c = 0; c < kprime; c++) out[c] = v[c].idx;
    qsort(out, (size_t)kprime, sizeof(int64_t), cmp_i64);
    free(qb); free(v);
    return ORC_OK;
}

/* ======================================================================== */
/* Self-Indexing workload.                                                   */
/* [SI] "Self-Indexing KVCache: Predicting Sparse Attention from Compressed  */
/* Keys" (gist.science/paper/2603.14224), Methodology A "One-Pass Sign-Based */
/* Vector Quantization", B "Compressed-Domain Top-k Retrieval (LUT-GEMV)",   */
/* C "Sink Tokens".                                                          */
/* ======================================================================== */

/* Prefill index of one (b, h).  Readings:                                  */
/*  - A.4 entropy-aware normalisation: the channel means are taken over the */
/*    indexed prefill keys [S, n) (the S sink tokens stay in full precision */
/*    and outside the index), sum in fp64 in key order, divided by the     */
/*    count in fp64, rounded once to fp32; n == S gives mean 0.            */
/*  - y = fp32(x - mean) for every key.                                     */
/*  - A.1/A.2 sub-vectors are the contiguous groups of 4 coordinates; the  */
/*    id of sub-vector b is sum_j [y_{4b+j} < 0] 2^j (zero on the + side). */
/*  - A.3 the centroid of cluster (b, p) is the mean of y_b over the        */
/*    prefill keys [S, n) with id_b = p (fp64 sum in key order / count,     */
/*    rounded once to fp32); an empty cluster has centroid 0.               */
/* ids [n][d/4] (every key gets ids), mean [d], cb [d/4][16][4].            */
int orc_si_build(int d, int64_t n, int64_t S, const float *X, float *mean,
                 uint8_t *ids, float *cb)
{
    if (d < 4 || d % 4 || n < 0 || S < 0) return ORC_EINVAL;
    int B = d / 4;
    int64_t m = n > S ? n - S : 0;
    for (int c = 0; c < d; c++) {
        double a = 0.0;
        for (int64_t i = S; i < n; i++) a += (double)X[i * d + c];
        mean[c] = m > 0 ? (float)(a / (double)m) : 0.0f;
    }
    for (int64_t i = 0; i < n; i++)
        for (int b = 0; b < B; b++) {
            unsigned id = 0;
            for (int j = 0; j < 4; j++) {
                float y = X[i * d + 4 * b + j] - mean[4 * b + j];
                if (y < 0.0f) id |= 1u << j;
            }
            ids[i * B + b] = (uint8_t)id;
        }
    double *sum = (double *)calloc((size_t)B * 64, sizeof(double));
    int64_t *cnt = (int64_t *)calloc((size_t)B * 16, sizeof(int64_t));
    if (!sum || !cnt) { free(sum); free(cnt); return ORC_EINVAL; }
    for (int64_t i = S; i < n; i++)
        for (int b = 0; b < B; b++) {
            int p = ids[i * B + b];
            cnt[b * 16 + p]++;
            for (int j = 0; j < 4; j++) {
                float y = X[i * d + 4 * b + j] - mean[4 * b + j];
                sum[(b * 16 + p) * 4 + j] += (double)y;
            }
        }
    for (int e = 0; e < B * 16; e++)
        for (int j = 0; j < 4; j++)
            cb[e * 4 + j] = cnt[e] ? (float)(sum[e * 4 + j] / (double)cnt[e]) : 0.0f;
    free(sum); free(cnt);
    return ORC_OK;
}

/* Sign ids of keys appended after the prefill, with the prefill means (the */
/* codebook is built once, in the prefill: [SI] Methodology A.3).           */
int orc_si_ids(int d, int64_t n, const float *X, const float *mean, uint8_t *ids)
{
    if (d < 4 || d % 4 || n < 0) return ORC_EINVAL;
    int B = d / 4;
    for (int64_t i = 0; i < n; i++)
        for (int b = 0; b < B; b++) {
            unsigned id = 0;
            for (int j = 0; j < 4; j++) {
                float y = X[i * d + 4 * b + j] - mean[4 * b + j];
                if (y < 0.0f) id |= 1u << j;
            }
            ids[i * B + b] = (uint8_t)id;
        }
    return ORC_OK;
}

/* [SI] Methodology B, the query's lookup table: the dot product of the     */
/* query sub-vector with each of the 16 centroids.  The query of a KV head  */
/* is the mean of its G query heads, as for ParisKV (fp32: q_0 + q_1 + ...  */
/* in head order, times fp32(1/G)).  lut[b][p] = ((0 + q_{4b} c_0) +        */
/* q_{4b+1} c_1) + ... in fp32.  The centring by the key means is left out  */
/* of the query side: it shifts every key's score by the same <q, mean>.   */
int orc_si_lut(int d, int G, const float *Q, const float *cb, float *lut)
{
    if (d < 4 || d % 4 || G < 1) return ORC_EINVAL;
    int B = d / 4;
    float invG = 1.0f / (float)G;
    for (int b = 0; b < B; b++) {
        float qb[4];
        for (int j = 0; j < 4; j++) {
            float acc = Q[4 * b + j];
            for (int g = 1; g < G; g++) acc = acc + Q[(int64_t)g * d + 4 * b + j];
            qb[j] = acc * invG;
        }
        for (int p = 0; p < 16; p++) {
            float s = 0.0f;
            for (int j = 0; j < 4; j++) s = s + qb[j] * cb[(b * 16 + p) * 4 + j];
            lut[b * 16 + p] = s;
        }
    }
    return ORC_OK;
}

/* [SI] Methodology B, the approximate score of a key: the sum of its LUT   */
/* entries, one per sub-vector, written out as that sum: fp32, sub-vectors  */
/* in order, s = 0; for b = 0 .. d/4 - 1: s = s + lut[b][id_b].  Scores of  */
/* keys [S, n).                                                              */
int orc_si_scores(int d, int64_t n, int64_t S, const uint8_t *ids,
                  const float *lut, float *scores)
{
    if (d < 4 || d % 4 || S < 0) return ORC_EINVAL;
    int B = d / 4;
    for (int64_t i = S; i < n; i++) {
        float s = 0.0f;
        for (int b = 0; b < B; b++) s = s + lut[b * 16 + ids[i * B + b]];
        scores[i - S] = s;
    }
    return ORC_OK;
}
