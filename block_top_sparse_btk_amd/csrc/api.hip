// C ABI of libbtk: host-side validation, launch planning and dispatch.
// Every argument is checked here before the first HIP call, so a rejected call
// has no side effects and the checks run on machines without a GPU.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

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

// Test hook of the decode step, read from the environment at each call (results
// never depend on it): BTK_STEP_TEST_FLAGS bit 0 makes every workgroup leave its
// own share for workgroup 0 and the workgroups without phase-2 items to claim,
// as if it had not started; with sketches, bit 1 takes the one-workgroup-per-unit
// kernel whenever its limits allow (however few the units), bit 2 never.
uint32_t env_u32(const char *name, uint32_t dflt) {
    const char *e = getenv(name);
    if (e && *e) {
        char *end = nullptr;
        const unsigned long v = strtoul(e, &end, 10);
        if (end && *end == 0 && v <= 0xffffffffUL) return (uint32_t)v;
    }
    return dflt;
}
uint32_t step_test_flags() { return env_u32("BTK_STEP_TEST_FLAGS", 0u) & 7u; }

}  // namespace

namespace btk {

WorkspaceLayout workspace_layout(const Dims &d, int top_k, bool dense) {
    const size_t units = (size_t)d.B * d.Hkv;
    const AttendPlan sp = plan_attend(d, top_k, false);
    const AttendPlan dp = plan_attend(d, d.max_blocks, true);
    const size_t nsplit =
        dense && dp.nsplit_max > sp.nsplit_max ? dp.nsplit_max : sp.nsplit_max;
    const size_t row = (size_t)d.group() * d.D + 2 * (size_t)d.group();
    WorkspaceLayout w;
    w.queue = kQueueOffset;
    w.claims = 256;
    w.state = w.claims + (size_t)2 * kMaxStepGrid * kClaimStride * sizeof(uint64_t);
    w.state_end = w.state + align256(units * kStateStride * sizeof(uint32_t));
    w.scores = 0;
    w.partials = align256(units * d.max_blocks * sizeof(float));
    w.scratch = w.partials + align256(units * nsplit * row * sizeof(float));
    w.sk_lo = w.sk_hi = 0;
    if (dense) {  // the sketch selection's interval ends
        w.sk_lo = w.scratch;
        w.sk_hi = w.sk_lo + align256(units * d.max_blocks * sizeof(float));
        w.scratch = w.sk_hi + align256(units * d.max_blocks * sizeof(float));
    }
    w.total = w.state_end + w.scratch;
    return w;
}

TokenWorkspaceLayout token_workspace_layout(const Dims &d, int top_tokens) {
    const size_t units = (size_t)d.B * d.Hkv;
    TokenWorkspaceLayout w;
    w.cap = top_tokens < d.max_blocks ? top_tokens : d.max_blocks;
    const AttendPlan ap = plan_attend(d, w.cap, false);
    const size_t row = (size_t)d.group() * d.D + 2 * (size_t)d.group();
    // the state lines where the block calls keep theirs, the scratch at the end
    w.state = 256 + (size_t)2 * kMaxStepGrid * kClaimStride * sizeof(uint64_t);
    w.state_end = w.state + align256(units * kStateStride * sizeof(uint32_t));
    w.scores = 0;
    w.entries = w.scores + align256(units * (size_t)d.max_blocks * kPage * sizeof(float));
    w.counts = w.entries + align256(units * (size_t)w.cap * sizeof(uint32_t));
    w.partials = w.counts + align256(units * sizeof(uint32_t));
    w.scratch = w.partials + align256(units * (size_t)ap.nsplit_max * row * sizeof(float));
    w.total = w.state_end + w.scratch;
    return w;
}

}  // namespace btk

extern "C" {

int btk_abi_version(void) { return BTK_ABI_VERSION; }

const char *btk_status_string(btk_status_t status) {
    // A C caller may pass any int here; in C++ an enum object holding a value
    // outside the enumerators' range is undefined, so read the bytes as an int.
    int s;
    memcpy(&s, &status, sizeof s);
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
    char *scratch = ws + w.scratch_at(workspace_bytes);
    float *sc = scores ? scores : reinterpret_cast<float *>(scratch + w.scores);
    uint32_t *state = reinterpret_cast<uint32_t *>(ws + w.state);
    const btk::SelectPlan plan = btk::plan_select(d);
    return hip_status(btk::launch_select(d, plan, q, centroids, block_table, seq_lens, top_k,
                                         indices, sc, state + btk::kStSelect,
                                         reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream));
}

size_t btk_sketch_bytes(const btk_problem_t *problem) {
    btk::Dims d;
    if (check_problem(problem, &d) != BTK_OK) return 0;
    return btk::sketch_bytes(d);
}

btk_status_t btk_sketch_update(const btk_problem_t *problem, const float *centroids,
                               const int32_t *block_table, const int32_t *seq_lens,
                               const int32_t *first_pos, void *sketch, size_t sketch_bytes,
                               void *workspace, size_t workspace_bytes, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!centroids || !block_table || !seq_lens || !sketch) return BTK_ERR_NULL;
    if (sketch_bytes < btk::sketch_bytes(d)) return BTK_ERR_WORKSPACE;
    // the error word only: any workspace of this problem
    const btk::WorkspaceLayout w = btk::workspace_layout(d, 1);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    return hip_status(btk::launch_sketch_update(d, centroids, block_table, seq_lens, first_pos,
                                                sketch, reinterpret_cast<uint32_t *>(workspace),
                                                (hipStream_t)stream));
}

btk_status_t btk_select_sketch(const btk_problem_t *problem, const void *q,
                               const float *centroids, const void *sketch, size_t sketch_bytes,
                               const int32_t *block_table, const int32_t *seq_lens,
                               int32_t top_k, int32_t *indices, void *workspace,
                               size_t workspace_bytes, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !centroids || !sketch || !block_table || !seq_lens || !indices)
        return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    if (sketch_bytes < btk::sketch_bytes(d)) return BTK_ERR_WORKSPACE;
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    char *scratch = ws + w.scratch_at(workspace_bytes);
    uint32_t *state = reinterpret_cast<uint32_t *>(ws + w.state);
    return hip_status(btk::launch_select_sketch(
        d, q, centroids, sketch, block_table, seq_lens, top_k, indices,
        reinterpret_cast<float *>(scratch + w.sk_lo), reinterpret_cast<float *>(scratch + w.sk_hi),
        reinterpret_cast<float *>(scratch + w.scores), state + btk::kStSelect,
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
    char *scratch = ws + w.scratch_at(workspace_bytes);
    float *sc = scores ? scores : reinterpret_cast<float *>(scratch + w.scores);
    uint32_t *state = reinterpret_cast<uint32_t *>(ws + w.state);
    return hip_status(btk::launch_select_shared(
        d, plan, pg, q, centroids, block_table, seq_lens, top_k, indices, sc,
        state + btk::kStSelect, state + btk::kStPrefix, reinterpret_cast<uint32_t *>(ws),
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
                                         reinterpret_cast<float *>(
                                             ws + w.scratch_at(workspace_bytes) + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.state) +
                                             btk::kStAttend,
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
                                         reinterpret_cast<float *>(
                                             ws + w.scratch_at(workspace_bytes) + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.state) +
                                             btk::kStAttend,
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
                                         reinterpret_cast<float *>(
                                             ws + w.scratch_at(workspace_bytes) + w.partials),
                                         reinterpret_cast<uint32_t *>(ws + w.state) +
                                             btk::kStAttend,
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
    char *scratch = ws + w.scratch_at(workspace_bytes);
    uint32_t *err = reinterpret_cast<uint32_t *>(ws);
    uint32_t *state = reinterpret_cast<uint32_t *>(ws + w.state);
    uint32_t *entries = reinterpret_cast<uint32_t *>(scratch + w.entries);
    uint32_t *counts = reinterpret_cast<uint32_t *>(scratch + w.counts);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = btk::launch_token_select(
        d, q, k_cache, block_table, seq_lens, top_tokens, w.cap,
        reinterpret_cast<float *>(scratch + w.scores), nullptr, entries, counts,
        state + btk::kStRange, token_indices, err, s);
    if (e != hipSuccess) return hip_status(e);
    const btk::AttendPlan plan = btk::plan_attend(d, w.cap, false);
    return hip_status(btk::launch_attend(d, plan, 3, q, k_cache, v_cache, block_table, seq_lens,
                                         reinterpret_cast<const int32_t *>(entries), w.cap, out,
                                         lse, reinterpret_cast<float *>(scratch + w.partials),
                                         state + btk::kStAttend, err, s, counts));
}

// ---- the allocation-free step: scratch in a library-owned device array

// One array per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[BTK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
// The array's state area: the header, the claim words and the state lines of
// at most kNoallocMaxUnits units (B * Hkv); every problem's scratch sits after
// it, in the array's last bytes.
constexpr size_t kNoallocMaxUnits = 16384;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, or NULL
bool g_scratch_clear[kMaxDevices];  // the state area still has to be cleared

// Zeroes [0, n) words (the scratch's state area on its first use on a device):
// a plain kernel, so that a caller may capture it in a graph.
__global__ void fill_zero_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

namespace btk {
size_t noalloc_state_bytes() {
    return 256 + (size_t)2 * kMaxStepGrid * kClaimStride * sizeof(uint64_t) +
           kNoallocMaxUnits * kStateStride * sizeof(uint32_t);
}
}  // namespace btk

// The single-launch step, with (k_new, v_new non-NULL) or without the KV append.
static btk_status_t decode_step(const btk_problem_t *problem, const void *q, const void *k_new,
                                const void *v_new, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *seq_lens,
                                const int32_t *first_pos, float *centroids, int32_t top_k,
                                int32_t *indices, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream, bool append,
                                bool own_scratch = false, void *sketch = nullptr,
                                size_t sketch_bytes = 0, int32_t *cand_counts = nullptr) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !centroids || !indices || !out)
        return BTK_ERR_NULL;
    if (append && (!k_new || !v_new)) return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    if (d.B > btk::kMaxStepBatch || !btk::step_rows_fit(d))
        return BTK_ERR_UNSUPPORTED;
    if (sketch && sketch_bytes < btk::sketch_bytes(d)) return BTK_ERR_WORKSPACE;
    // a caller's workspace has the size btk_workspace_bytes promises; the
    // library's own scratch holds only what the step needs
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k, !own_scratch);
    if (!workspace || workspace_bytes < w.total) return BTK_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    char *scratch = ws + w.scratch_at(workspace_bytes);
    uint32_t *state = reinterpret_cast<uint32_t *>(ws + w.state);
    const btk::SelectPlan sp = btk::plan_select(d);
    const btk::AttendPlan ap = btk::plan_attend(d, top_k, false);
    return hip_status(btk::launch_decode_step(
        d, sp, ap, q, k_cache, v_cache, block_table, seq_lens, first_pos, centroids, top_k,
        indices, reinterpret_cast<float *>(scratch + w.scores), out, lse,
        reinterpret_cast<float *>(scratch + w.partials), state + btk::kStSelect,
        state + btk::kStAttend, state + btk::kStReady, reinterpret_cast<uint32_t *>(ws + w.queue),
        reinterpret_cast<uint32_t *>(ws + btk::kStealOffset),
        reinterpret_cast<unsigned long long *>(ws + w.claims), btk::kReadySpinLimit,
        step_test_flags(),
        reinterpret_cast<uint32_t *>(ws), (hipStream_t)stream, append ? k_new : nullptr,
        append ? v_new : nullptr, sketch,
        sketch ? reinterpret_cast<float *>(scratch + w.sk_lo) : nullptr,
        sketch ? reinterpret_cast<float *>(scratch + w.sk_hi) : nullptr, cand_counts));
}

btk_status_t btk_decode_step_sketch(const btk_problem_t *problem, const void *q,
                                    const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens,
                                    const int32_t *first_pos, float *centroids, void *sketch,
                                    size_t sketch_bytes, int32_t top_k, int32_t *indices,
                                    void *out, float *lse, int32_t *cand_counts, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (!sketch) return BTK_ERR_NULL;
    return decode_step(problem, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens,
                       first_pos, centroids, top_k, indices, out, lse, workspace,
                       workspace_bytes, stream, false, false, sketch, sketch_bytes, cand_counts);
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

btk_status_t btk_decode_step_noalloc(const btk_problem_t *problem, const void *q,
                                     const void *k_cache, const void *v_cache,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     const int32_t *first_pos, float *centroids, int32_t top_k,
                                     int32_t *indices, void *out, float *lse, void *stream) {
    btk::Dims d;
    btk_status_t st = check_problem(problem, &d);
    if (st != BTK_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !centroids || !indices || !out)
        return BTK_ERR_NULL;
    if (!top_k_ok(top_k)) return BTK_ERR_SHAPE;
    if (d.B > btk::kMaxStepBatch || !btk::step_rows_fit(d)) return BTK_ERR_UNSUPPORTED;
    // the step's own layout: no room for the dense comparison's partials
    const btk::WorkspaceLayout w = btk::workspace_layout(d, top_k, false);
    if ((size_t)d.B * d.Hkv > kNoallocMaxUnits ||
        w.scratch > (size_t)BTK_NOALLOC_SCRATCH_BYTES - btk::noalloc_state_bytes())
        return BTK_ERR_WORKSPACE;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return BTK_ERR_UNSUPPORTED;
    void *ws = nullptr;
    bool clear = false;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e);
            if (!p) return BTK_ERR_HIP;
            g_scratch_ptr[dev] = p;
            g_scratch_clear[dev] = true;
        }
        ws = g_scratch_ptr[dev];
        clear = g_scratch_clear[dev];
        g_scratch_clear[dev] = false;
    }
    if (clear) {  // every word that carries state from call to call starts at zero
        const size_t words = btk::noalloc_state_bytes() / sizeof(uint32_t);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream,
                           static_cast<uint32_t *>(ws), words);
        e = hipGetLastError();
        if (e != hipSuccess) {
            std::lock_guard<std::mutex> lock(g_scratch_mu);
            g_scratch_clear[dev] = true;
            return hip_status(e);
        }
    }
    return decode_step(problem, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens,
                       first_pos, centroids, top_k, indices, out, lse, ws,
                       (size_t)BTK_NOALLOC_SCRATCH_BYTES, stream, false, true);
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

btk_status_t btk_probe_row_read(const void *src, size_t src_bytes, const int32_t *row_ids,
                               int64_t rows, uint32_t *sink, void *stream) {
    if (!src || !sink) return BTK_ERR_NULL;
    const int64_t src_rows = (int64_t)(src_bytes / 512);
    if (rows < 0 || (!row_ids && rows > src_rows)) return BTK_ERR_SHAPE;
    if (rows == 0) return BTK_OK;
    return hip_status(btk::launch_row_read_probe(src, src_rows, row_ids, rows, sink,
                                                 (hipStream_t)stream));
}

}  // extern "C"
