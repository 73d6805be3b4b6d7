// Internal declarations shared by the HIP translation units of libbtk.
// Device helpers for gfx950 (wave64, MFMA), the launch plans that the C ABI
// computes on the host, and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace btk {

constexpr int kWave = 64;
constexpr int kPage = 16;           // tokens per page (block); all kernels assume it
constexpr int kMaxBlocksPerSeq = 8192;  // select holds one key per block in LDS
constexpr int kMaxGroup = 16;       // query heads per KV head: MFMA tile rows
constexpr int kMaxStepBatch = 1024; // decode step: per-sequence item prefix kept in LDS
constexpr int kMaxTopTokens = kMaxBlocksPerSeq * kPage;  // token-level baseline budget
// Shared-prefix selection: prefix blocks per shared item.  Each of its rows is
// scored against every member's mean query, so items are kept short to spread
// that arithmetic over many workgroups (each row is still read once).
constexpr int kSharedChunk = 32;

// error bits in workspace word 0
constexpr uint32_t kErrSeqLen = 1u;
constexpr uint32_t kErrPage = 2u;
constexpr uint32_t kErrIndex = 4u;
constexpr uint32_t kErrTimeout = 8u;  // decode step: a wait for published data gave up
constexpr uint32_t kErrPrefix = 16u;  // a declared shared prefix differs between members

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;

// ---- device helpers ------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// float -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Order-preserving map of a float score to uint32 (larger score -> larger key);
// -0.0 maps like +0.0 so that the two tie.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void store_relaxed(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_relaxed(const float *p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ void store_relaxed_i32(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int32_t load_relaxed_i32(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_relaxed_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-workgroup hand-off without L2 maintenance.  Every value another
// workgroup reads is written with store_relaxed and read with load_relaxed:
// agent-scope atomic accesses, which gfx950 performs coherently across the
// XCDs' L2 caches.  A workgroup publishes by waiting until its own such stores
// have completed, then counting itself in with an agent-scope atomic; the one
// that brings the count to `total` sees every other workgroup's stores with its
// own load_relaxed reads.  A device-scope __threadfence() would instead write
// back and invalidate the whole L2 of the XCD in every workgroup.
// Returns true in all threads of the last workgroup, which also re-arms the
// counter to zero for the next launch.
__device__ __forceinline__ bool arrive_last(uint32_t *counter, uint32_t total, int *flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = prev == total - 1;
        if (prev == total - 1)
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return *flag != 0;
}

__device__ __forceinline__ void flag_error(uint32_t *err, uint32_t bit) {
    if (err) atomicOr(err, bit);
}

// ---- launch plans ----------------------------------------------------------

struct Dims {
    int B, Hq, Hkv, D, num_pages, max_blocks, dtype;
    float sm_scale;  // resolved (> 0)
    int group() const { return Hq / Hkv; }
};

struct SelectPlan {
    int chunk;       // blocks scored per workgroup
    int nchunk_max;  // chunks per unit at max_blocks
};

struct AttendPlan {
    int bps;         // list entries (blocks) per workgroup split
    int nsplit_max;  // splits per unit at the longest list
};

SelectPlan plan_select(const Dims &d);

// Best-of-N groups for the shared-prefix selection: sequences [start[g],
// start[g+1]) share their first blocks[g] block-table entries; item0[g] is the
// first shared-scoring workgroup of group g (item0[n] = their number).  Small
// enough to travel as a kernel argument.
constexpr int kMaxPrefixGroups = 64;
constexpr int kMaxGroupMembers = 32;
struct PrefixGroups {
    int n;
    int start[kMaxPrefixGroups + 1];
    int blocks[kMaxPrefixGroups];
    int item0[kMaxPrefixGroups + 1];
};
AttendPlan plan_attend(const Dims &d, int list_len_max, bool dense);

// Workspace layout (bytes, each region 256-aligned):
//   [0, 256)                   error word; decode-step chunk counter at byte kStealOffset
//                              and queue words at byte kQueueOffset
//   shared-prefix flags        kMaxPrefixGroups*Hkv*2 uint32   zero after every call
//   select counters            B*Hkv uint32      zero after every call
//   attend counters            B*Hkv uint32      zero after every call
//   ready words                B*Hkv*kReadyStride uint32 (decode step: launch tags)
//   scores scratch             B*Hkv*max_blocks float
//   attend partials            B*Hkv*nsplit_max*(r*D + 2r) float (max of sparse, dense)
// Every region that carries state from call to call comes before the scratch,
// the ones left at zero first and the tags next, and each grows with B*Hkv: a
// smaller problem on the same workspace then finds zeros where it needs zeros
// and, where it reads tags, only zeros or tags of earlier launches.
constexpr int kReadyStride = 32;     // one 128-byte line per unit: each is polled on its own
constexpr size_t kQueueOffset = 128;  // 4 uint32: spare, exits, launch counter, spare
constexpr size_t kStealOffset = 64;   // 1 uint32, off the queue words' line
struct WorkspaceLayout {
    size_t pflags, sel_counters, att_counters, scores, partials, ready, queue, total;
};
WorkspaceLayout workspace_layout(const Dims &d, int top_k);

// ---- launchers (return hipError_t of the launch) --------------------------

hipError_t launch_centroid_update(const Dims &d, const void *k_cache, const int32_t *block_table,
                                  const int32_t *seq_lens, const int32_t *first_pos,
                                  float *centroids, hipStream_t stream);

hipError_t launch_select(const Dims &d, const SelectPlan &plan, const void *q,
                         const float *centroids, const int32_t *block_table,
                         const int32_t *seq_lens, int top_k, int32_t *indices, float *scores,
                         uint32_t *counters, uint32_t *err, hipStream_t stream);

// mode: 0 the selected blocks, 1 every block, 2 the most recent min(top_k, n_b),
// 3 counts[unit] packed entries (block | token mask << 16) in `indices`, top_k
// being the list capacity
// S2+S3 with the shared prefixes of `pg` scored once per (group, KV head):
// results identical to launch_select.
hipError_t launch_select_shared(const Dims &d, const SelectPlan &plan, const PrefixGroups &pg,
                                const void *q, const float *centroids,
                                const int32_t *block_table, const int32_t *seq_lens, int top_k,
                                int32_t *indices, float *scores, uint32_t *counters,
                                uint32_t *pflags, uint32_t *err, hipStream_t stream);

hipError_t launch_attend(const Dims &d, const AttendPlan &plan, int mode, const void *q,
                         const void *k_cache, const void *v_cache, const int32_t *block_table,
                         const int32_t *seq_lens, const int32_t *indices, int top_k, void *out,
                         float *lse, float *partials, uint32_t *counters, uint32_t *err,
                         hipStream_t stream, const uint32_t *counts = nullptr);

// Token-level baseline: scores of every valid token, then per unit the
// top_tokens best as packed entries (cap = min(max_blocks, top_tokens) per unit)
// with their count, and token positions when token_idx is not NULL.
hipError_t launch_token_select(const Dims &d, const void *q, const void *k_cache,
                               const int32_t *block_table, const int32_t *seq_lens,
                               int top_tokens, int cap, float *scores, uint32_t *counters,
                               uint32_t *entries, uint32_t *counts, uint32_t *ranges,
                               int32_t *token_idx, uint32_t *err, hipStream_t stream);

// Workspace of the token-level baseline (bytes, each region 256-aligned):
//   [0, 256) error word; counters; score ranges B*Hkv*2 uint32; attend counters
//   (these three zero after every call); counts B*Hkv uint32; scores
//   B*Hkv*max_blocks*16 float; entries B*Hkv*cap uint32; partials
struct TokenWorkspaceLayout {
    size_t counters, scores, entries, counts, ranges, att_counters, partials, total;
    int cap;
};
TokenWorkspaceLayout token_workspace_layout(const Dims &d, int top_tokens);

// Whether the decode step's row count (every unit charged a fixed number of
// rows beyond its blocks) fits its 32-bit counters.
bool step_rows_fit(const Dims &d);
hipError_t launch_decode_step(const Dims &d, const SelectPlan &sp, const AttendPlan &ap,
                              const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *first_pos, float *centroids, int top_k,
                              int32_t *indices, float *scores, void *out, float *lse,
                              float *partials, uint32_t *sel_counters, uint32_t *att_counters,
                              uint32_t *ready, uint32_t *queue, uint32_t *steal,
                              uint32_t *err, hipStream_t stream,
                              const void *k_new = nullptr, const void *v_new = nullptr);

}  // namespace btk
