/*
 * oracle.c -- plain, slow CPU reference for block top-k sparse decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (sources are the pages on the Kinetics paper):
 *   - "Pith review of 'Kinetics: Rethinking Test-Time Scaling Laws'"
 *     (pith.science), section "What carries the argument": block top-k attention
 *     summarises each block of keys by its averaged key vector, scores the blocks
 *     with the queries of one query group (the r query heads of a grouped-query
 *     attention group), keeps the k best blocks per group and attends only to them.
 *   - "Kinetics README" (GitLite mirror), section "Benchmark Block TopK Attention
 *     throughput": the KV cache is paged, a block is one page (16 tokens in the
 *     example command), and top-k is counted in pages.
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   group score = mean over the group's heads of the scaled logit against the
 *   centroid; scale = 1/sqrt(D) unless given; a partial last block is a candidate
 *   and its centroid averages only its valid tokens; ties go to the lower logical
 *   block index; selected indices are emitted in ascending order, -1 padded;
 *   no forced blocks; query head h uses KV head h / r.
 *
 * Precision: inputs are read exactly (bf16 bit patterns or fp32), every sum is
 * taken in double, and values that the method stores (centroids, block scores)
 * are rounded to float, so the selection decision is taken on fp32 scores.
 * Attention is evaluated in double and returned rounded to float.
 *
 * Layouts (all row-major, host memory):
 *   q          [B][Hq][D]
 *   k_cache    [num_pages][Hkv][P][D]      (token-major pages)
 *   v_cache    [num_pages][Hkv][D][P]      (dim-major pages)
 *   block_table[B][max_blocks] int32, seq_lens[B] int32 (>= 1, counts the newest token)
 *   centroids  [num_pages][Hkv][D] float
 *   scores     [B][Hkv][max_blocks] float
 *   indices    [B][Hkv][top_k] int32
 *   out        [B][Hq][D] float, lse [B][Hq] float
 *
 * Parallelism: OpenMP over independent (sequence, KV head) units or pages; each
 * unit's arithmetic is the same sequential loop at any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_DATA = 2, OR_ERR_NOMEM = 3 };
enum { OR_BF16 = 0, OR_F32 = 1 };

/* ---- element access --------------------------------------------------- */

static double elem(const void *base, int dtype, size_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[i];
    /* bf16 is the upper half of an IEEE binary32 pattern: widening is exact. */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t k_index(int page, int g, int t, int d, int Hkv, int P, int D)
{
    return (((size_t)page * Hkv + g) * P + t) * D + d;
}

static size_t v_index(int page, int g, int t, int d, int Hkv, int P, int D)
{
    return (((size_t)page * Hkv + g) * D + d) * P + t;
}

/* number of blocks of a sequence of L tokens, and the valid tokens of block j */
static int n_blocks(int L, int P) { return (L + P - 1) / P; }
static int valid_in_block(int L, int P, int j)
{
    int v = L - j * P;
    return v < P ? v : P;
}

static double resolve_scale(double sm_scale, int D)
{
    return sm_scale > 0.0 ? sm_scale : 1.0 / sqrt((double)D);
}

static int check_tables(int B, int P, int num_pages, int max_blocks,
                        const int32_t *block_table, const int32_t *seq_lens)
{
    for (int b = 0; b < B; ++b) {
        int L = seq_lens[b];
        if (L < 1 || L > max_blocks * P)
            return OR_ERR_DATA;
        for (int j = 0; j < n_blocks(L, P); ++j) {
            int page = block_table[(size_t)b * max_blocks + j];
            if (page < 0 || page >= num_pages)
                return OR_ERR_DATA;
        }
    }
    return OR_OK;
}

int oracle_abi_version(void) { return 1; }

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- centroids: the averaged key vector of each block ------------------
 * For every page touched by a sequence (all of its blocks, or only the blocks
 * holding positions first_pos[b] .. L_b-1 when first_pos is given), and every
 * KV head g:  c[page][g][:] = float( (sum over the valid tokens t of K_t) / v ).
 * A page referenced by several sequences must have the same valid-token count
 * in each of them (shared prompt pages are full); otherwise OR_ERR_DATA.
 */
int oracle_centroids(int dtype, int B, int Hkv, int D, int P, int num_pages,
                     int max_blocks, const void *k_cache,
                     const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *first_pos, float *centroids)
{
    if (B < 1 || Hkv < 1 || D < 1 || P < 1 || num_pages < 1 || max_blocks < 1 ||
        !k_cache || !block_table || !seq_lens || !centroids ||
        (dtype != OR_BF16 && dtype != OR_F32))
        return OR_ERR_ARG;
    int rc = check_tables(B, P, num_pages, max_blocks, block_table, seq_lens);
    if (rc)
        return rc;

    /* valid-token count of each page to rebuild; 0 = leave untouched */
    int *need = (int *)calloc((size_t)num_pages, sizeof(int));
    if (!need)
        return OR_ERR_NOMEM;
    for (int b = 0; b < B && rc == OR_OK; ++b) {
        int L = seq_lens[b];
        int j0 = 0;
        if (first_pos) {
            if (first_pos[b] < 0 || first_pos[b] >= L) {
                rc = OR_ERR_DATA;
                break;
            }
            j0 = first_pos[b] / P;
        }
        for (int j = j0; j < n_blocks(L, P); ++j) {
            int page = block_table[(size_t)b * max_blocks + j];
            int v = valid_in_block(L, P, j);
            if (need[page] != 0 && need[page] != v) {
                rc = OR_ERR_DATA;
                break;
            }
            need[page] = v;
        }
    }
    if (rc == OR_OK) {
#pragma omp parallel for schedule(dynamic, 16)
        for (long pg = 0; pg < (long)num_pages * Hkv; ++pg) {
            int page = (int)(pg / Hkv), g = (int)(pg % Hkv);
            int v = need[page];
            if (v == 0)
                continue;
            for (int d = 0; d < D; ++d) {
                double sum = 0.0;
                for (int t = 0; t < v; ++t)
                    sum += elem(k_cache, dtype, k_index(page, g, t, d, Hkv, P, D));
                centroids[((size_t)page * Hkv + g) * D + d] = (float)(sum / v);
            }
        }
    }
    free(need);
    return rc;
}

/* ---- block scores -------------------------------------------------------
 * s[b][g][j] = float( (1/r) * sum over the r query heads h of group g of
 *              scale * sum_d q[b][h][d] * c[bt[b][j]][g][d] ),   j < n_b.
 * Entries j >= n_b are not written.
 */
int oracle_scores(int dtype, int B, int Hq, int Hkv, int D, int P, int num_pages,
                  int max_blocks, const void *q, const float *centroids,
                  const int32_t *block_table, const int32_t *seq_lens,
                  double sm_scale, float *scores)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || P < 1 || num_pages < 1 ||
        max_blocks < 1 || !q || !centroids || !block_table || !seq_lens || !scores ||
        (dtype != OR_BF16 && dtype != OR_F32))
        return OR_ERR_ARG;
    int rc = check_tables(B, P, num_pages, max_blocks, block_table, seq_lens);
    if (rc)
        return rc;
    const int r = Hq / Hkv;
    const double scale = resolve_scale(sm_scale, D);

#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < (long)B * Hkv; ++u) {
        int b = (int)(u / Hkv), g = (int)(u % Hkv);
        int nb = n_blocks(seq_lens[b], P);
        for (int j = 0; j < nb; ++j) {
            int page = block_table[(size_t)b * max_blocks + j];
            const float *c = centroids + ((size_t)page * Hkv + g) * D;
            double group = 0.0;
            for (int h = g * r; h < (g + 1) * r; ++h) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += elem(q, dtype, ((size_t)b * Hq + h) * D + d) * (double)c[d];
                group += scale * dot;
            }
            scores[((size_t)b * Hkv + g) * max_blocks + j] = (float)(group / r);
        }
    }
    return OR_OK;
}

/* ---- top-k selection ----------------------------------------------------
 * Rank blocks j < n_b by (score descending, j ascending); keep the first
 * k_b = min(top_k, n_b); write them in ascending j, then -1 for the rest.
 * Scores are compared as floats (so -0.0 and +0.0 tie).  NaN scores are an error.
 */
typedef struct {
    float s;
    int j;
} ranked_t;

static int rank_cmp(const void *pa, const void *pb)
{
    const ranked_t *a = (const ranked_t *)pa, *b = (const ranked_t *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int int_cmp(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    return (a > b) - (a < b);
}

int oracle_select(int B, int Hkv, int P, int max_blocks, const float *scores,
                  const int32_t *seq_lens, int top_k, int32_t *indices)
{
    if (B < 1 || Hkv < 1 || P < 1 || max_blocks < 1 || top_k < 1 || !scores ||
        !seq_lens || !indices)
        return OR_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 1 || seq_lens[b] > max_blocks * P)
            return OR_ERR_DATA;
    int rc = OR_OK;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
    for (long u = 0; u < (long)B * Hkv; ++u) {
        int b = (int)(u / Hkv);
        int nb = n_blocks(seq_lens[b], P);
        const float *s = scores + (size_t)u * max_blocks;
        int32_t *out = indices + (size_t)u * top_k;
        ranked_t *rk = (ranked_t *)malloc(sizeof(ranked_t) * (size_t)nb);
        int *keep = (int *)malloc(sizeof(int) * (size_t)nb);
        if (!rk || !keep) {
            free(rk);
            free(keep);
            rc |= OR_ERR_NOMEM;
            continue;
        }
        int bad = 0;
        for (int j = 0; j < nb; ++j) {
            if (isnan(s[j]))
                bad = 1;
            rk[j].s = s[j];
            rk[j].j = j;
        }
        if (bad) {
            free(rk);
            free(keep);
            rc |= OR_ERR_DATA;
            continue;
        }
        qsort(rk, (size_t)nb, sizeof(ranked_t), rank_cmp);
        int kb = top_k < nb ? top_k : nb;
        for (int i = 0; i < kb; ++i)
            keep[i] = rk[i].j;
        qsort(keep, (size_t)kb, sizeof(int), int_cmp);
        for (int i = 0; i < top_k; ++i)
            out[i] = i < kb ? keep[i] : -1;
        free(rk);
        free(keep);
    }
    return rc;
}

/* ---- exact softmax attention over a block set ---------------------------
 * For query head h of sequence b (KV head g = h / r), the token set T is every
 * valid token of the listed blocks (indices[b][g][:], -1 entries ignored), or
 * of all blocks when indices is NULL.  With l_t = scale * q_h . K_t,
 * m = max l, w_t = exp(l_t - m), Z = sum w:
 *     out_h = sum_t (w_t / Z) V_t,   lse_h = m + ln Z.
 * weights (optional) receives w_t / Z at the token's logical position in
 * [B][Hq][max_blocks * P], zero elsewhere.  A listed block must be < n_b and
 * listed once (OR_ERR_DATA otherwise); an empty set is an error.
 */
int oracle_attend(int dtype, int B, int Hq, int Hkv, int D, int P, int num_pages,
                  int max_blocks, const void *q, const void *k_cache,
                  const void *v_cache, const int32_t *block_table,
                  const int32_t *seq_lens, const int32_t *indices, int top_k,
                  double sm_scale, float *out, float *lse, double *weights)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || P < 1 || num_pages < 1 ||
        max_blocks < 1 || !q || !k_cache || !v_cache || !block_table || !seq_lens ||
        !out || (indices && top_k < 1) || (dtype != OR_BF16 && dtype != OR_F32))
        return OR_ERR_ARG;
    int rc = check_tables(B, P, num_pages, max_blocks, block_table, seq_lens);
    if (rc)
        return rc;
    const int r = Hq / Hkv;
    const double scale = resolve_scale(sm_scale, D);
    const size_t max_tok = (size_t)max_blocks * P;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
    for (long bh = 0; bh < (long)B * Hq; ++bh) {
        int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / r;
        int L = seq_lens[b], nb = n_blocks(L, P);

        /* the block list, in the order given (ascending for the dense case) */
        int *blocks = (int *)malloc(sizeof(int) * (size_t)(nb > 0 ? nb : 1));
        char *seen = (char *)calloc((size_t)nb, 1);
        double *logit = (double *)malloc(sizeof(double) * (size_t)L);
        int *tok_block = (int *)malloc(sizeof(int) * (size_t)L);
        int *tok_slot = (int *)malloc(sizeof(int) * (size_t)L);
        double *acc = (double *)calloc((size_t)D, sizeof(double));
        if (!blocks || !seen || !logit || !tok_block || !tok_slot || !acc) {
            rc |= OR_ERR_NOMEM;
            goto done;
        }
        int nsel = 0;
        if (indices) {
            const int32_t *sel = indices + ((size_t)b * Hkv + g) * top_k;
            for (int i = 0; i < top_k; ++i) {
                int j = sel[i];
                if (j < 0)
                    continue;
                if (j >= nb || seen[j]) {
                    rc |= OR_ERR_DATA;
                    goto done;
                }
                seen[j] = 1;
                blocks[nsel++] = j;
            }
        } else {
            for (int j = 0; j < nb; ++j)
                blocks[nsel++] = j;
        }
        if (nsel == 0) {
            rc |= OR_ERR_DATA;
            goto done;
        }

        /* logits of every gathered token */
        int ntok = 0;
        double m = -INFINITY;
        for (int i = 0; i < nsel; ++i) {
            int j = blocks[i];
            int page = block_table[(size_t)b * max_blocks + j];
            for (int t = 0; t < valid_in_block(L, P, j); ++t) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += elem(q, dtype, ((size_t)b * Hq + h) * D + d) *
                           elem(k_cache, dtype, k_index(page, g, t, d, Hkv, P, D));
                logit[ntok] = scale * dot;
                tok_block[ntok] = j;
                tok_slot[ntok] = t;
                if (logit[ntok] > m)
                    m = logit[ntok];
                ++ntok;
            }
        }
        /* softmax weights and the weighted sum of values */
        double Z = 0.0;
        for (int i = 0; i < ntok; ++i) {
            logit[i] = exp(logit[i] - m); /* logit[] now holds w_t */
            Z += logit[i];
        }
        for (int i = 0; i < ntok; ++i) {
            int j = tok_block[i], t = tok_slot[i];
            int page = block_table[(size_t)b * max_blocks + j];
            double w = logit[i] / Z;
            for (int d = 0; d < D; ++d)
                acc[d] += w * elem(v_cache, dtype, v_index(page, g, t, d, Hkv, P, D));
            if (weights)
                weights[((size_t)b * Hq + h) * max_tok + (size_t)j * P + t] = w;
        }
        for (int d = 0; d < D; ++d)
            out[((size_t)b * Hq + h) * D + d] = (float)acc[d];
        if (lse)
            lse[(size_t)b * Hq + h] = (float)(m + log(Z));
    done:
        free(blocks);
        free(seen);
        free(logit);
        free(tok_block);
        free(tok_slot);
        free(acc);
    }
    return rc;
}

/* ---- output rounding: float -> bf16, round to nearest, ties to even ------ */
void oracle_round_bf16(const float *in, uint16_t *out, long n)
{
    for (long i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &in[i], sizeof u);
        if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
            out[i] = (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
            continue;
        }
        uint32_t lsb = (u >> 16) & 1u;
        u += 0x7fffu + lsb;
        out[i] = (uint16_t)(u >> 16);
    }
}
