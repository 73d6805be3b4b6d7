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
constexpr int kMaxStepBatch = 65536; // decode step: batch limit (one LDS row per 1024 sequences)
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

// Device code handles vectors only as clang's native vector types (indexed with
// [], converted with __builtin_bit_cast), never as HIP's float4 / uint4 structs
// accessed through their .x .. .w union members or through pointers of another
// type: a build of the fp32 attention with one-block stages, written with those,
// had the P.V fragments' registers reused before the products read them.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// Element e of a 16-byte vector of T held as raw bits (8 bf16 or 4 fp32), as float.
template <typename T>
__device__ __forceinline__ float vec16_elem(const u32x4_t &w, int e);

// ---- device helpers ------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

template <>
__device__ __forceinline__ float vec16_elem<uint16_t>(const u32x4_t &w, int e) {
    return bf16_bits_to_f32((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
}
template <>
__device__ __forceinline__ float vec16_elem<float>(const u32x4_t &w, int e) {
    return __uint_as_float(w[e]);
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
AttendPlan plan_attend(const Dims &d, int list_len_max, bool dense, int target = 256);

// Workspace layout (bytes).  Everything that carries state from call to call
// sits at the start, at places that do not depend on the problem; the scratch
// of a call (values written before they are read) sits at the END of the
// workspace the caller passes.  So a workspace sized for a problem serves any
// problem whose unit count (B*Hkv) and sizes are at most those: its state words
// are where the larger problem's are, and its scratch never reaches them.
//   [0, 256)                   error word; decode-step chunk counter at byte kStealOffset
//                              and queue words at byte kQueueOffset
//   decode-step claim words    2*kMaxStepGrid*kClaimStride uint64 (the bank the next
//                              launch uses is zero after every call)
//   state lines                B*Hkv lines of kStateStride uint32 (one 128-byte line per
//                              unit u, each polled or counted on its own): kStReady the
//                              decode step's launch tag, kStSelect / kStAttend the select /
//                              attention arrival counters, kStPrefix two shared-prefix
//                              flags of (group, KV head) u = group*Hkv + head, kStRange
//                              two score-range words of the token-level path; all zero
//                              after every call but the tags
//   ... unused ...
//   scores scratch             B*Hkv*max_blocks float        } the last bytes of the
//   attend partials            B*Hkv*nsplit_max*(r*D + 2r) float } workspace
// (partials: max of the sparse and the dense plan; the sparse plan only for the
// decode step's own layout).
constexpr int kStateStride = 32;
constexpr int kStReady = 0, kStSelect = 1, kStAttend = 2, kStPrefix = 3, kStRange = 5;
constexpr int kReadyStride = kStateStride;
constexpr size_t kQueueOffset = 128;  // 4 uint32: spare, exits, launch counter, claim bank
constexpr size_t kStealOffset = 64;   // 1 uint32 (decode-step chunk counter), off the queue line
// Decode step: share claims, one 64-bit word per workgroup share (a 64-byte line
// each), in two banks that alternate from launch to launch; grids are capped at
// kMaxStepGrid workgroups.
constexpr int kMaxStepGrid = 2048;
constexpr int kClaimStride = 8;       // 64-bit words
// Bound of a decode-step wait for a unit's scores (polls, ~0.1 s; a safeguard:
// every wait ends well before).
constexpr uint32_t kReadySpinLimit = 1u << 22;
struct WorkspaceLayout {
    size_t claims, state, queue;  // offsets from the start
    size_t scores, partials;      // offsets from the start of the scratch
    size_t sk_lo, sk_hi;          // the sketch selection's interval ends (full layout only)
    size_t state_end, scratch, total;
    // the scratch's offset in a workspace of `bytes` bytes (>= total): its last
    // `scratch` bytes, 256-aligned
    size_t scratch_at(size_t bytes) const { return (bytes - scratch) & ~(size_t)255; }
};
WorkspaceLayout workspace_layout(const Dims &d, int top_k, bool dense = true);

// Block sketches (sketch.hip): bytes of a problem's sketch, where its code rows
// start, the sketch update and the selection that uses it.
size_t sketch_bytes(const Dims &d);
size_t sketch_rows_offset(const Dims &d);
hipError_t launch_sketch_update(const Dims &d, const float *centroids, const int32_t *block_table,
                                const int32_t *seq_lens, const int32_t *first_pos, void *sketch,
                                uint32_t *err, hipStream_t stream);
hipError_t launch_select_sketch(const Dims &d, const void *q, const float *centroids,
                                const void *sketch, const int32_t *block_table,
                                const int32_t *seq_lens, int top_k, int32_t *indices,
                                float *lo, float *hi, float *exact, uint32_t *counters,
                                uint32_t *err, hipStream_t stream);

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

// Workspace of the token-level baseline: the header, the claim words and the
// state lines as above (kStRange and kStAttend used), and at its end the
// scratch: scores B*Hkv*max_blocks*16 float, entries B*Hkv*cap uint32, counts
// B*Hkv uint32, partials.
struct TokenWorkspaceLayout {
    size_t state;                               // offset from the start (state lines)
    size_t scores, entries, counts, partials;   // offsets from the start of the scratch
    size_t state_end, scratch, total;
    int cap;
    size_t scratch_at(size_t bytes) const { return (bytes - scratch) & ~(size_t)255; }
};
TokenWorkspaceLayout token_workspace_layout(const Dims &d, int top_tokens);

// Whether the persistent decode step's row count (every unit charged a fixed
// number of rows beyond its blocks) fits its 32-bit counters.
bool step_rows_fit(const Dims &d);
hipError_t launch_decode_step(const Dims &d, const SelectPlan &sp, const AttendPlan &ap,
                              const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *first_pos, float *centroids, int top_k,
                              int32_t *indices, float *scores, void *out, float *lse,
                              float *partials, uint32_t *sel_counters, uint32_t *att_counters,
                              uint32_t *ready, uint32_t *queue, uint32_t *steal,
                              unsigned long long *claims, uint32_t spin_limit,
                              uint32_t test_flags, uint32_t *err, hipStream_t stream,
                              const void *k_new = nullptr, const void *v_new = nullptr,
                              void *sketch = nullptr, float *sk_lo = nullptr,
                              float *sk_hi = nullptr, int32_t *cand_counts = nullptr);

// Counter calibration (probe.hip): reads `rows` 512-byte rows of src (row ids
// from row_ids, or 0 .. rows-1 when it is NULL; ids outside [0, src_rows) are
// skipped) with 16 bytes per lane.
hipError_t launch_row_read_probe(const void *src, int64_t src_rows, const int32_t *row_ids,
                                 int64_t rows, uint32_t *sink, hipStream_t stream);

}  // namespace btk
