// C ABI of libbtk: host-side validation, launch planning and dispatch.
// Every argument is checked here before the first HIP call, so a rejected call
// has no side effects and the checks run on machines without a GPU.
#include <math.h>

#include "btk.h"
#include "btk_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

btk_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return BTK_OK;
    g_last_hip_error = (int)e;
    return BTK_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Validates the problem; fills the internal dims on success.
btk_status_t check_problem(const btk_problem_t *p, btk::Dims *d) {
    if (!p) return BTK_ERR_NULL;
    if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 ||
        p->page_size < 1 || p->num_pages < 1 || p->max_blocks_per_seq < 1)
        return BTK_ERR_SHAPE;
    if (p->num_q_heads % p->num_kv_heads) return BTK_ERR_SHAPE;
    if (!(isfinite(p->sm_scale))) return BTK_ERR_SHAPE;
    if (p->dtype != BTK_BF16 && p->dtype != BTK_F32) return BTK_ERR_UNSUPPORTED;
    if (p->head_dim != 64 && p->head_dim != 128) return BTK_ERR_UNSUPPORTED;
    if (p->page_size != btk::kPage) return BTK_ERR_UNSUPPORTED;
    if (p->num_q_heads / p->num_kv_heads > btk::kMaxGroup) return BTK_ERR_UNSUPPORTED;
    if (p->max_blocks_per_seq > btk::kMaxBlocksPerSeq) return BTK_ERR_UNSUPPORTED;
    // grid sizes stay well inside 32 bits
    if ((size_t)p->batch * p->num_kv_heads * p->max_blocks_per_seq > ((size_t)1 << 31))
        return BTK_ERR_UNSUPPORTED;
    d->B = p->batch;
    d->Hq = p->num_q_heads;
    d->Hkv = p->num_kv_heads;
    d->D = p->head_dim;
    d->num_pages = p->num_pages;
    d->max_blocks = p->max_blocks_per_seq;
    d->dtype = p->dtype;
    d->sm_scale = p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
    return BTK_OK;
}

bool top_k_ok(int32_t top_k) { return top_k >= 1 && top_k <= btk::kMaxBlocksPerSeq; }

}  // namespace

namespace btk {

WorkspaceLayout workspace_layout(const Dims &d, int top_k) {
    const size_t units = (size_t)d.B * d.Hkv;
    const AttendPlan sp = plan_attend(d, top_k, false);
    const AttendPlan dp = plan_attend(d, d.max_blocks, true);
    const size_t nsplit = sp.nsplit_max > dp.nsplit_max ? sp.nsplit_max : dp.nsplit_max;
    const size_t row = (size_t)d.group() * d.D + 2 * (size_t)d.group();
    WorkspaceLayout w;
    w.queue = kQueueOffset;
    w.pflags = 256;
    w.sel_counters = w.pflags + align256((size_t)kMaxPrefixGroups * d.Hkv * 2 * sizeof(uint32_t));
    w.att_counters = w.sel_counters + align256(units * sizeof(uint32_t));
    w.ready = w.att_counters + align256(units * sizeof(uint32_t));
    w.scores = w.ready + align256(units * (size_t)kReadyStride * sizeof(uint32_t));
    w.partials = w.scores + align256(units * d.max_blocks * sizeof(float));
    w.total = w.partials + align256(units * nsplit * row * sizeof(float));
    return w;
}

TokenWorkspaceLayout token_workspace_layout(const Dims &d, int top_tokens) {
    const size_t units = (size_t)d.B * d.Hkv;
    TokenWorkspaceLayout w;
    w.cap = top_tokens < d.max_blocks ? top_tokens : d.max_blocks;
    const AttendPlan ap = plan_attend(d, w.cap, false);
    const size_t row = (size_t)d.group() * d.D + 2 * (size_t)d.group();
    // state kept from call to call (all zero after a call) first, then scratch,
    // so that a smaller problem on the same workspace finds zeros there
    w.counters = 256;
    w.ranges = w.counters + align256(units * sizeof(uint32_t));
    w.att_counters = w.ranges + align256(2 * units * sizeof(uint32_t));
    w.counts = w.att_counters + align256(units * sizeof(uint32_t));
    w.scores = w.counts + align256(units * sizeof(uint32_t));
    w.entries = w.scores + align256(units * (size_t)d.max_blocks * kPage * sizeof(float));
    w.partials = w.entries + align256(units * (size_t)w.cap * sizeof(uint32_t));
    w.total = w.partials + align256(units * (size_t)ap.nsplit_max * row * sizeof(float));
    return w;
}

}  // namespace btk

extern "C" {

int btk_abi_version(void) { return BTK_ABI_VERSION; }

const char *btk_status_string(btk_status_t s) {
    switch (s) {
    case BTK_OK: return "ok";
    case BTK_ERR_NULL: return "a required pointer is NULL";
    case BTK_ERR_SHAPE: return "a size is out of range or inconsistent";
    case BTK_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, page_size or limit";
    case BTK_ERR_WORKSPACE: return "workspace missing or too small";
    case BTK_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

int btk_last_hip_error(void) { return g_last_hip_error; }

size_t btk_workspace_bytes(const btk_problem_t *problem, int32_t top_k) {
    btk::Dims d;
    if (check_problem(problem, &d) != BTK_OK || !top_k_ok(top_k)) return 0;
    return btk::workspace_layout(d, top_k).total;
}

btk_status_t btk_centroid_update(const btk_problem_t *problem, const void *k_cache,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 const int32_t *first_pos, float *centroids, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!k_cache || !block_table || !seq_lens || !centroids) return BTK_ERR_NULL;
    return hip_status(btk::launch_centroid_update(d, k_cache, block_table, seq_lens, first_pos,
                                                  centroids, (hipStream_t)stream));
}

btk_status_t btk_select(const btk_problem_t *problem, const void *q, const float *centroids,
                        const int32_t *block_table, const int32_t *seq_lens, int32_t top_k,
                        int32_t *indices, float *scores, void *workspace,
                        size_t workspace_bytes, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !centroids || !block_table || !seq_lens || !indices) return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    float *sc = scores ? scores : reinterpret_cast<float *>(ws + w.scores);
    const btk::SelectPlan plan = btk::plan_select(d);
    return hip_status(btk::launch_select(d, plan, q, centroids, block_table, seq_lens, top_k,
                                         indices, sc,
                                         reinterpret_cast<uint32_t *>(ws + w.sel_counters),
                                         reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream));
}

btk_status_t btk_select_shared(const btk_problem_t *problem, const void *q,
                               const float *centroids, const int32_t *block_table,
                               const int32_t *seq_lens, int32_t num_groups,
                               const int32_t *group_start, const int32_t *prefix_blocks,
                               int32_t top_k, int32_t *indices, float *scores, void *workspace,
                               size_t workspace_bytes, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !centroids || !block_table || !seq_lens || !indices || !group_start ||
        !prefix_blocks)
        return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    if (num_groups < 1 || num_groups > btk::kMaxPrefixGroups) return BTK_ERR_UNSUPPORTED;
    const btk::SelectPlan plan = btk::plan_select(d);
    btk::PrefixGroups pg{};
    pg.n = num_groups;
    if (group_start[0] < 0) return BTK_ERR_SHAPE;
    for (int g = 0; g < num_groups; ++g) {
        const int a0 = group_start[g], a1 = group_start[g + 1];
        if (a1 <= a0 || a1 > d.B) return BTK_ERR_SHAPE;
        if (a1 - a0 > btk::kMaxGroupMembers) return BTK_ERR_UNSUPPORTED;
        if (prefix_blocks[g] < 0 || prefix_blocks[g] > d.max_blocks) return BTK_ERR_SHAPE;
        pg.start[g] = a0;
        pg.blocks[g] = prefix_blocks[g];
        pg.item0[g + 1] = pg.item0[g] + d.Hkv * ((prefix_blocks[g] + btk::kSharedChunk - 1) /
                                                 btk::kSharedChunk);
    }
    pg.start[num_groups] = group_start[num_groups];
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    float *sc = scores ? scores : reinterpret_cast<float *>(ws + w.scores);
    return hip_status(btk::launch_select_shared(
        d, plan, pg, q, centroids, block_table, seq_lens, top_k, indices, sc,
        reinterpret_cast<uint32_t *>(ws + w.sel_counters),
        reinterpret_cast<uint32_t *>(ws + w.pflags), reinterpret_cast<uint32_t *>(ws),
        (hipStream_t)stream));
}

btk_status_t btk_sparse_attend(const btk_problem_t *problem, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_table,
                               const int32_t *seq_lens, const int32_t *indices, int32_t top_k,
                               void *out, float *lse, void *workspace, size_t workspace_bytes,
                               void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !indices || !out)
        return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const btk::AttendPlan plan = btk::plan_attend(d, top_k, false);
    return hip_status(btk::launch_attend(d, plan, 0, q, k_cache, v_cache, block_table,
                                         seq_lens, indices, top_k, out, lse,
                                         reinterpret_cast<float *>(ws + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.att_counters),
                                         reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream));
}

btk_status_t btk_dense_attend(const btk_problem_t *problem, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, void *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return BTK_ERR_NULL;
    // the dense path needs no top_k; size the workspace as for top_k = 1
    const btk::WorkspaceLayout w = btk::workspace_layout(d, 1);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const btk::AttendPlan plan = btk::plan_attend(d, d.max_blocks, true);
    return hip_status(btk::launch_attend(d, plan, 1, q, k_cache, v_cache, block_table,
                                         seq_lens, nullptr, 0, out, lse,
                                         reinterpret_cast<float *>(ws + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.att_counters),
                                         reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream));
}

btk_status_t btk_local_attend(const btk_problem_t *problem, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, int32_t window_blocks, void *out,
                              float *lse, void *workspace, size_t workspace_bytes,
                              void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return BTK_ERR_NULL;
    if (!top_k_ok(window_blocks)) return BTK_ERR_SHAPE;
    const btk::WorkspaceLayout w = btk::workspace_layout(d, window_blocks);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const btk::AttendPlan plan = btk::plan_attend(d, window_blocks, false);
    return hip_status(btk::launch_attend(d, plan, 2, q, k_cache, v_cache, block_table,
                                         seq_lens, nullptr, window_blocks, out, lse,
                                         reinterpret_cast<float *>(ws + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.att_counters),
                                         reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream));
}

size_t btk_token_workspace_bytes(const btk_problem_t *problem, int32_t top_tokens) {
    btk::Dims d;
    if (check_problem(problem, &d) != BTK_OK || top_tokens < 1 || top_tokens > btk::kMaxTopTokens)
        return 0;
    return btk::token_workspace_layout(d, top_tokens).total;
}

btk_status_t btk_token_topk_attend(const btk_problem_t *problem, const void *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *block_table, const int32_t *seq_lens,
                                   int32_t top_tokens, int32_t *token_indices, void *out,
                                   float *lse, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return BTK_ERR_NULL;
    if (top_tokens < 1 || top_tokens > btk::kMaxTopTokens) return BTK_ERR_SHAPE;
    const btk::TokenWorkspaceLayout w = btk::token_workspace_layout(d, top_tokens);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    uint32_t *err = reinterpret_cast<uint32_t *>(ws);
    uint32_t *entries = reinterpret_cast<uint32_t *>(ws + w.entries);
    uint32_t *counts = reinterpret_cast<uint32_t *>(ws + w.counts);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = btk::launch_token_select(
        d, q, k_cache, block_table, seq_lens, top_tokens, w.cap,
        reinterpret_cast<float *>(ws + w.scores), reinterpret_cast<uint32_t *>(ws + w.counters),
        entries, counts, reinterpret_cast<uint32_t *>(ws + w.ranges), token_indices, err, s);
    if (e != hipSuccess) return hip_status(e);
    const btk::AttendPlan plan = btk::plan_attend(d, w.cap, false);
    return hip_status(btk::launch_attend(d, plan, 3, q, k_cache, v_cache, block_table, seq_lens,
                                         reinterpret_cast<const int32_t *>(entries), w.cap, out,
                                         lse, reinterpret_cast<float *>(ws + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.att_counters), err,
                                         s, counts));
}

// The single-launch step, with (k_new, v_new non-NULL) or without the KV append.
static btk_status_t decode_step(const btk_problem_t *problem, const void *q, const void *k_new,
                                const void *v_new, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *seq_lens,
                                const int32_t *first_pos, float *centroids, int32_t top_k,
                                int32_t *indices, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream, bool append) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !centroids || !indices || !out)
        return BTK_ERR_NULL;
    if (append && (!k_new || !v_new)) return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    if (d.B > btk::kMaxStepBatch || !btk::step_rows_fit(d)) return BTK_ERR_UNSUPPORTED;
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const btk::SelectPlan sp = btk::plan_select(d);
    const btk::AttendPlan ap = btk::plan_attend(d, top_k, false);
    return hip_status(btk::launch_decode_step(
        d, sp, ap, q, k_cache, v_cache, block_table, seq_lens, first_pos, centroids, top_k,
        indices, reinterpret_cast<float *>(ws + w.scores), out, lse,
        reinterpret_cast<float *>(ws + w.partials),
        reinterpret_cast<uint32_t *>(ws + w.sel_counters),
        reinterpret_cast<uint32_t *>(ws + w.att_counters),
        reinterpret_cast<uint32_t *>(ws + w.ready), reinterpret_cast<uint32_t *>(ws + w.queue),
        reinterpret_cast<uint32_t *>(ws + btk::kStealOffset),
        reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream, append ? k_new : nullptr,
        append ? v_new : nullptr));
}

btk_status_t btk_decode_step(const btk_problem_t *problem, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *seq_lens, const int32_t *first_pos, float *centroids,
                             int32_t top_k, int32_t *indices, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream) {
    return decode_step(problem, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens,
                       first_pos, centroids, top_k, indices, out, lse, workspace,
                       workspace_bytes, stream, false);
}

btk_status_t btk_decode_step_append(const btk_problem_t *problem, const void *q,
                                    const void *k_new, const void *v_new, void *k_cache,
                                    void *v_cache, const int32_t *block_table,
                                    const int32_t *seq_lens, float *centroids, int32_t top_k,
                                    int32_t *indices, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return decode_step(problem, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                       nullptr, centroids, top_k, indices, out, lse, workspace, workspace_bytes,
                       stream, true);
}

}  // extern "C"
