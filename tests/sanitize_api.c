/*
 * Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * library's host side (test infrastructure; built and run by
 * tests/test_sanitizers.py, on a machine without a GPU).  Every entry point is
 * called with arguments it must reject before any HIP call: a NULL or
 * inconsistent problem, extreme sizes, NULL buffers, top_k out of range, a
 * workspace one byte short, malformed prefix groups in exactly sized host
 * arrays.  Device pointers are dummies that the host never dereferences.  The
 * size queries run over a sweep of valid and invalid problems.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "btk.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const int got_ = (int)(call);                                                   \
        if (got_ != (int)(want)) {                                                      \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
                    (int)(want));                                                       \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

static btk_problem_t base(void) {
    btk_problem_t p = {4, 32, 8, 128, 16, 4096, 512, BTK_BF16, 0.0f};
    return p;
}

int main(void) {
    void *dev = (void *)(uintptr_t)0x10000; /* never dereferenced on the host */
    const int32_t *di = (const int32_t *)dev;
    int32_t *wi = (int32_t *)dev;
    float *wf = (float *)dev;
    btk_problem_t p = base();

    EXPECT(btk_abi_version(), BTK_ABI_VERSION);
    for (int s = -1; s <= 6; ++s)
        if (!btk_status_string((btk_status_t)s)) ++failures;

    /* size queries over valid and invalid problems */
    const int32_t bs[] = {-1, 0, 1, 3, 1024, 4096, INT_MAX};
    const int32_t hs[] = {0, 1, 3, 8, 32, 64, 17};
    const int32_t ds[] = {0, 63, 64, 128, 256};
    const int32_t ms[] = {-5, 0, 1, 2047, 8192, 8193, INT_MAX};
    const int32_t ks[] = {-1, 0, 1, 64, 8192, 8193, INT_MAX};
    for (unsigned a = 0; a < sizeof bs / sizeof bs[0]; ++a)
        for (unsigned b = 0; b < sizeof hs / sizeof hs[0]; ++b)
            for (unsigned c = 0; c < sizeof ds / sizeof ds[0]; ++c)
                for (unsigned e = 0; e < sizeof ms / sizeof ms[0]; ++e)
                    for (unsigned f = 0; f < sizeof ks / sizeof ks[0]; ++f) {
                        btk_problem_t q = base();
                        q.batch = bs[a];
                        q.num_kv_heads = hs[b];
                        q.num_q_heads = hs[b] * 4;
                        q.head_dim = ds[c];
                        q.max_blocks_per_seq = ms[e];
                        q.dtype = (a + f) & 1;
                        const size_t w = btk_workspace_bytes(&q, ks[f]);
                        const size_t t = btk_token_workspace_bytes(&q, ks[f] == INT_MAX ? INT_MAX : ks[f] * 16);
                        const int ok = bs[a] >= 1 && hs[b] >= 1 && (ds[c] == 64 || ds[c] == 128) &&
                                       ms[e] >= 1 && ms[e] <= 8192 &&
                                       (double)bs[a] * hs[b] * ms[e] <= 2147483648.0;
                        if ((ok && ks[f] >= 1 && ks[f] <= 8192) != (w != 0)) {
                            fprintf(stderr, "workspace_bytes(%d,%d,%d,%d,%d) = %zu\n", bs[a], hs[b],
                                    ds[c], ms[e], ks[f], w);
                            ++failures;
                        }
                        if (!ok && t != 0) ++failures;
                    }
    EXPECT(btk_workspace_bytes(NULL, 8), 0);
    p.sm_scale = NAN;
    EXPECT(btk_workspace_bytes(&p, 8), 0);
    p.sm_scale = INFINITY;
    EXPECT(btk_workspace_bytes(&p, 8), 0);
    p = base();
    p.num_q_heads = 30; /* not a multiple of num_kv_heads */
    EXPECT(btk_workspace_bytes(&p, 8), 0);
    p.num_q_heads = 8 * 17; /* group of 17 */
    EXPECT(btk_workspace_bytes(&p, 8), 0);
    p = base();
    p.page_size = 32;
    EXPECT(btk_workspace_bytes(&p, 8), 0);
    p = base();
    p.dtype = 7;
    EXPECT(btk_workspace_bytes(&p, 8), 0);

    p = base();
    const size_t need = btk_workspace_bytes(&p, 64);
    if (need == 0) ++failures;
    void *ws = dev;

    /* S1 */
    EXPECT(btk_centroid_update(NULL, dev, di, di, NULL, wf, NULL), BTK_ERR_NULL);
    EXPECT(btk_centroid_update(&p, NULL, di, di, NULL, wf, NULL), BTK_ERR_NULL);
    EXPECT(btk_centroid_update(&p, dev, di, di, NULL, NULL, NULL), BTK_ERR_NULL);
    /* S2 + S3 */
    EXPECT(btk_select(&p, dev, wf, di, di, 64, wi, NULL, NULL, need, NULL), BTK_ERR_WORKSPACE);
    EXPECT(btk_select(&p, dev, wf, di, di, 64, wi, NULL, ws, need - 1, NULL), BTK_ERR_WORKSPACE);
    EXPECT(btk_select(&p, dev, wf, di, di, 0, wi, NULL, ws, need, NULL), BTK_ERR_SHAPE);
    EXPECT(btk_select(&p, dev, wf, di, di, 8193, wi, NULL, ws, need, NULL), BTK_ERR_SHAPE);
    EXPECT(btk_select(&p, NULL, wf, di, di, 64, wi, NULL, ws, need, NULL), BTK_ERR_NULL);
    EXPECT(btk_select(&p, dev, wf, di, di, 64, NULL, NULL, ws, need, NULL), BTK_ERR_NULL);

    /* prefix groups in exactly sized host arrays */
    int32_t *gs = malloc(3 * sizeof(int32_t)), *pb = malloc(2 * sizeof(int32_t));
    gs[0] = 0; gs[1] = 2; gs[2] = 4; pb[0] = 10; pb[1] = 512;
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, gs, pb, 64, wi, NULL, ws, need - 1, NULL),
           BTK_ERR_WORKSPACE);
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 0, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_UNSUPPORTED);
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 65, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_UNSUPPORTED);
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, NULL, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_NULL);
    pb[1] = 513;
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    pb[1] = -1;
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    pb[1] = 512;
    gs[2] = 5; /* past the batch */
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    gs[1] = 0; gs[2] = 4; /* empty group */
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    gs[0] = -1;
    EXPECT(btk_select_shared(&p, dev, wf, di, di, 2, gs, pb, 64, wi, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    free(gs);
    free(pb);
    {
        btk_problem_t big = base();
        big.batch = 40;
        const size_t nb = btk_workspace_bytes(&big, 64);
        int32_t *g1 = malloc(2 * sizeof(int32_t)), *p1 = malloc(sizeof(int32_t));
        g1[0] = 0; g1[1] = 33; p1[0] = 4; /* 33 members */
        EXPECT(btk_select_shared(&big, dev, wf, di, di, 1, g1, p1, 64, wi, NULL, ws, nb, NULL),
               BTK_ERR_UNSUPPORTED);
        free(g1);
        free(p1);
    }

    /* S4, S5 and the baselines */
    EXPECT(btk_sparse_attend(&p, dev, dev, dev, di, di, di, 64, dev, NULL, ws, need - 1, NULL),
           BTK_ERR_WORKSPACE);
    EXPECT(btk_sparse_attend(&p, dev, dev, dev, di, di, NULL, 64, dev, NULL, ws, need, NULL),
           BTK_ERR_NULL);
    EXPECT(btk_sparse_attend(&p, dev, dev, dev, di, di, di, -3, dev, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    {
        const size_t nd = btk_workspace_bytes(&p, 1);
        EXPECT(btk_dense_attend(&p, dev, dev, dev, di, di, dev, NULL, NULL, nd, NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_dense_attend(&p, dev, dev, NULL, di, di, dev, NULL, ws, nd, NULL), BTK_ERR_NULL);
    }
    EXPECT(btk_local_attend(&p, dev, dev, dev, di, di, 0, dev, NULL, ws, need, NULL), BTK_ERR_SHAPE);
    EXPECT(btk_local_attend(&p, dev, dev, dev, di, di, 64, dev, NULL, ws, need - 1, NULL),
           BTK_ERR_WORKSPACE);
    {
        const size_t nt = btk_token_workspace_bytes(&p, 1024);
        if (nt == 0) ++failures;
        EXPECT(btk_token_workspace_bytes(&p, 0), 0);
        EXPECT(btk_token_workspace_bytes(&p, 131073), 0);
        EXPECT(btk_token_topk_attend(&p, dev, dev, dev, di, di, 1024, NULL, dev, NULL, ws, nt - 1,
                                     NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_token_topk_attend(&p, dev, dev, dev, di, di, 131073, NULL, dev, NULL, ws, nt,
                                     NULL),
               BTK_ERR_SHAPE);
        EXPECT(btk_token_topk_attend(&p, dev, NULL, dev, di, di, 1024, NULL, dev, NULL, ws, nt,
                                     NULL),
               BTK_ERR_NULL);
    }

    /* single-launch step, its fused-append form and its allocation-free form */
    EXPECT(btk_decode_step(&p, dev, dev, dev, di, di, di, wf, 64, wi, dev, NULL, ws, need - 1, NULL),
           BTK_ERR_WORKSPACE);
    EXPECT(btk_decode_step(&p, dev, dev, dev, di, di, di, NULL, 64, wi, dev, NULL, ws, need, NULL),
           BTK_ERR_NULL);
    EXPECT(btk_decode_step(&p, dev, dev, dev, di, di, di, wf, 0, wi, dev, NULL, ws, need, NULL),
           BTK_ERR_SHAPE);
    EXPECT(btk_decode_step_append(&p, dev, NULL, dev, dev, dev, di, di, wf, 64, wi, dev, NULL, ws,
                                  need, NULL),
           BTK_ERR_NULL);
    EXPECT(btk_decode_step_append(&p, dev, dev, dev, dev, dev, di, di, wf, 64, wi, dev, NULL, ws,
                                  need - 1, NULL),
           BTK_ERR_WORKSPACE);
    {
        btk_problem_t big = base();
        big.batch = 65537;
        const size_t nb = btk_workspace_bytes(&big, 64);
        EXPECT(btk_decode_step(&big, dev, dev, dev, di, di, di, wf, 64, wi, dev, NULL, ws, nb, NULL),
               BTK_ERR_UNSUPPORTED);
        EXPECT(btk_decode_step_noalloc(&big, dev, dev, dev, di, di, di, wf, 64, wi, dev, NULL, NULL),
               BTK_ERR_UNSUPPORTED);
        big.batch = 1024;
        big.num_kv_heads = 32; /* 32768 units: more than the array's state lines */
        big.num_q_heads = 32;
        big.max_blocks_per_seq = 16;
        EXPECT(btk_decode_step_noalloc(&big, dev, dev, dev, di, di, di, wf, 8, wi, dev, NULL, NULL),
               BTK_ERR_WORKSPACE);
        big = base();
        big.batch = 512;
        big.max_blocks_per_seq = 8192; /* scores alone exceed the array */
        EXPECT(btk_decode_step_noalloc(&big, dev, dev, dev, di, di, di, wf, 64, wi, dev, NULL, NULL),
               BTK_ERR_WORKSPACE);
    }
    EXPECT(btk_decode_step_noalloc(NULL, dev, dev, dev, di, di, di, wf, 64, wi, dev, NULL, NULL),
           BTK_ERR_NULL);
    EXPECT(btk_decode_step_noalloc(&p, dev, dev, dev, di, di, di, wf, 64, NULL, dev, NULL, NULL),
           BTK_ERR_NULL);
    EXPECT(btk_decode_step_noalloc(&p, dev, dev, dev, di, di, di, wf, 9000, wi, dev, NULL, NULL),
           BTK_ERR_SHAPE);

    /* block sketches */
    {
        const size_t sk = btk_sketch_bytes(&p);
        if (sk == 0) ++failures;
        EXPECT(btk_sketch_bytes(NULL), 0);
        EXPECT(btk_sketch_update(&p, wf, di, di, NULL, NULL, sk, ws, need, NULL), BTK_ERR_NULL);
        EXPECT(btk_sketch_update(&p, wf, di, di, NULL, dev, sk - 1, ws, need, NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_sketch_update(&p, wf, di, di, NULL, dev, sk, NULL, need, NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_select_sketch(&p, dev, wf, dev, sk, di, di, 0, wi, ws, need, NULL),
               BTK_ERR_SHAPE);
        EXPECT(btk_select_sketch(&p, dev, wf, NULL, sk, di, di, 64, wi, ws, need, NULL),
               BTK_ERR_NULL);
        EXPECT(btk_select_sketch(&p, dev, wf, dev, sk - 1, di, di, 64, wi, ws, need, NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_select_sketch(&p, dev, wf, dev, sk, di, di, 64, wi, ws, need - 1, NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_decode_step_sketch(NULL, dev, dev, dev, di, di, di, wf, dev, sk, 64, wi, dev,
                                      NULL, NULL, ws, need, NULL),
               BTK_ERR_NULL);
        EXPECT(btk_decode_step_sketch(&p, dev, dev, dev, di, di, di, wf, NULL, sk, 64, wi, dev,
                                      NULL, NULL, ws, need, NULL),
               BTK_ERR_NULL);
        EXPECT(btk_decode_step_sketch(&p, dev, dev, dev, di, di, di, wf, dev, sk, 0, wi, dev,
                                      NULL, NULL, ws, need, NULL),
               BTK_ERR_SHAPE);
        EXPECT(btk_decode_step_sketch(&p, dev, dev, dev, di, di, di, wf, dev, sk - 1, 64, wi, dev,
                                      NULL, NULL, ws, need, NULL),
               BTK_ERR_WORKSPACE);
        EXPECT(btk_decode_step_sketch(&p, dev, dev, dev, di, di, di, wf, dev, sk, 64, wi, dev,
                                      NULL, NULL, ws, need - 1, NULL),
               BTK_ERR_WORKSPACE);
    }

    /* counter-calibration probe */
    EXPECT(btk_probe_row_read(NULL, 4096, NULL, 8, (uint32_t *)dev, NULL), BTK_ERR_NULL);
    EXPECT(btk_probe_row_read(dev, 4096, NULL, 8, NULL, NULL), BTK_ERR_NULL);
    EXPECT(btk_probe_row_read(dev, 4096, NULL, -1, (uint32_t *)dev, NULL), BTK_ERR_SHAPE);
    EXPECT(btk_probe_row_read(dev, 4096, NULL, 9, (uint32_t *)dev, NULL), BTK_ERR_SHAPE);
    EXPECT(btk_probe_row_read(dev, 4096, di, -5, (uint32_t *)dev, NULL), BTK_ERR_SHAPE);
    EXPECT(btk_probe_row_read(dev, 4096, NULL, 0, (uint32_t *)dev, NULL), BTK_OK);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("api sanitizer driver: ok\n");
    return 0;
}
