/*
 * Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU
 * oracle (test infrastructure; built and run by tests/test_sanitizers.py).
 * Calls every oracle entry point on small ragged inputs (fp32 and bf16,
 * partial last blocks, k >= n_b, decode-position updates, attention weights)
 * and on inputs it must reject, and checks return codes and a few properties
 * (selection rows ascending and -1 padded, softmax weights summing to 1).
 * Input values come from a fixed linear congruential sequence.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_centroids(int dtype, int B, int Hkv, int D, int P, int num_pages, int max_blocks,
                     const void *k_cache, const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *first_pos, float *centroids);
int oracle_scores(int dtype, int B, int Hq, int Hkv, int D, int P, int num_pages, int max_blocks,
                  const void *q, const float *centroids, const int32_t *block_table,
                  const int32_t *seq_lens, double sm_scale, float *scores);
int oracle_select(int B, int Hkv, int P, int max_blocks, const float *scores,
                  const int32_t *seq_lens, int top_k, int32_t *indices);
int oracle_attend(int dtype, int B, int Hq, int Hkv, int D, int P, int num_pages, int max_blocks,
                  const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_table, const int32_t *seq_lens, const int32_t *indices,
                  int top_k, double sm_scale, float *out, float *lse, double *weights);
void oracle_round_bf16(const float *in, uint16_t *out, long n);

static uint32_t rng = 12345u;
static float draw(void) {
    rng = rng * 1664525u + 1013904223u;
    return (float)((rng >> 8) & 0xffff) / 32768.0f - 1.0f;
}

static int failures = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static void run(int dtype, int D, int r, int Hkv, const int *lens, int B, int top_k) {
    const int P = 16, Hq = r * Hkv;
    int max_blocks = 0, num_pages = 1;
    for (int b = 0; b < B; ++b) {
        const int nb = (lens[b] + P - 1) / P;
        if (nb > max_blocks) max_blocks = nb;
        num_pages += nb;
    }
    const size_t esz = dtype ? 4 : 2;
    const size_t kn = (size_t)num_pages * Hkv * P * D;
    void *k = malloc(kn * esz), *v = malloc(kn * esz), *q = malloc((size_t)B * Hq * D * esz);
    float *tmp = malloc(kn * sizeof(float));
    for (size_t i = 0; i < kn; ++i) tmp[i] = draw();
    if (dtype) memcpy(k, tmp, kn * 4); else oracle_round_bf16(tmp, k, (long)kn);
    for (size_t i = 0; i < kn; ++i) tmp[i] = draw();
    if (dtype) memcpy(v, tmp, kn * 4); else oracle_round_bf16(tmp, v, (long)kn);
    for (size_t i = 0; i < (size_t)B * Hq * D; ++i) tmp[i] = draw();
    if (dtype) memcpy(q, tmp, (size_t)B * Hq * D * 4);
    else oracle_round_bf16(tmp, q, (long)((size_t)B * Hq * D));
    int32_t *bt = malloc(sizeof(int32_t) * B * max_blocks), *sl = malloc(sizeof(int32_t) * B);
    int32_t *fp = malloc(sizeof(int32_t) * B);
    int page = 1;  /* page 0 is never referenced */
    for (int b = 0; b < B; ++b) {
        const int nb = (lens[b] + P - 1) / P;
        for (int j = 0; j < max_blocks; ++j) bt[b * max_blocks + j] = j < nb ? page + j : 0;
        page += nb;
        sl[b] = lens[b];
        fp[b] = lens[b] - 1;
    }
    float *cent = calloc((size_t)num_pages * Hkv * D, sizeof(float));
    float *sc = malloc(sizeof(float) * B * Hkv * max_blocks);
    int32_t *idx = malloc(sizeof(int32_t) * B * Hkv * top_k);
    float *out = malloc(sizeof(float) * B * Hq * D), *lse = malloc(sizeof(float) * B * Hq);
    double *w = calloc((size_t)B * Hq * max_blocks * P, sizeof(double));

    CHECK(oracle_centroids(dtype, B, Hkv, D, P, num_pages, max_blocks, k, bt, sl, NULL, cent) == 0);
    CHECK(oracle_centroids(dtype, B, Hkv, D, P, num_pages, max_blocks, k, bt, sl, fp, cent) == 0);
    CHECK(oracle_scores(dtype, B, Hq, Hkv, D, P, num_pages, max_blocks, q, cent, bt, sl, 0.0, sc) == 0);
    CHECK(oracle_select(B, Hkv, P, max_blocks, sc, sl, top_k, idx) == 0);
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g) {
            const int nb = (lens[b] + P - 1) / P, kb = top_k < nb ? top_k : nb;
            const int32_t *row = idx + ((size_t)b * Hkv + g) * top_k;
            for (int i = 0; i < top_k; ++i) {
                if (i < kb) CHECK(row[i] >= 0 && row[i] < nb && (i == 0 || row[i] > row[i - 1]));
                else CHECK(row[i] == -1);
            }
        }
    CHECK(oracle_attend(dtype, B, Hq, Hkv, D, P, num_pages, max_blocks, q, k, v, bt, sl, idx, top_k,
                        0.07, out, lse, w) == 0);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            double s = 0.0;
            for (int t = 0; t < max_blocks * P; ++t) s += w[((size_t)b * Hq + h) * max_blocks * P + t];
            CHECK(fabs(s - 1.0) < 1e-9);
            CHECK(isfinite(lse[b * Hq + h]));
        }
    CHECK(oracle_attend(dtype, B, Hq, Hkv, D, P, num_pages, max_blocks, q, k, v, bt, sl, NULL, 0,
                        0.0, out, lse, NULL) == 0);
    /* rejected inputs: bad shapes, NULLs, a page id past the pool, a length beyond the table */
    CHECK(oracle_centroids(dtype, 0, Hkv, D, P, num_pages, max_blocks, k, bt, sl, NULL, cent) != 0);
    CHECK(oracle_scores(dtype, B, Hkv > 1 ? Hq + 1 : 0, Hkv, D, P, num_pages, max_blocks, q, cent, bt, sl, 0.0, sc) != 0);
    CHECK(oracle_select(B, Hkv, P, max_blocks, NULL, sl, top_k, idx) != 0);
    CHECK(oracle_select(B, Hkv, P, max_blocks, sc, sl, 0, idx) != 0);
    bt[0] = num_pages + 5;
    CHECK(oracle_centroids(dtype, B, Hkv, D, P, num_pages, max_blocks, k, bt, sl, NULL, cent) != 0);
    CHECK(oracle_attend(dtype, B, Hq, Hkv, D, P, num_pages, max_blocks, q, k, v, bt, sl, NULL, 0, 0.0,
                        out, lse, NULL) != 0);
    bt[0] = 1;
    sl[0] = max_blocks * P + 1;
    CHECK(oracle_scores(dtype, B, Hq, Hkv, D, P, num_pages, max_blocks, q, cent, bt, sl, 0.0, sc) != 0);
    free(k); free(v); free(q); free(tmp); free(bt); free(sl); free(fp); free(cent); free(sc);
    free(idx); free(out); free(lse); free(w);
}

int main(void) {
    const int lens1[] = {1, 17, 300, 33};
    const int lens2[] = {1000, 16, 15, 513};
    run(1, 64, 2, 1, lens1, 4, 3);
    run(0, 128, 4, 2, lens2, 4, 8);
    run(0, 64, 1, 3, lens1, 4, 40);  /* k >= n_b everywhere */
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
