// Single-launch decode step: S1 (touched pages) + S2 + S3 + S4 in one persistent
// kernel.  (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What
// carries the argument": averaged-key block summaries, per-query-group scoring,
// top-k blocks, attention over the kept blocks.)
//
// Work items come from a queue counter in the workspace, in this order:
//   1. scoring items, one per (sequence, KV head, chunk), unit-major with a
//      unit's chunks from last to first: the chunk that holds a touched page
//      first recomputes its centroid, then the chunk is scored; the workgroup
//      that completes the unit (a counter per unit) selects its top-k blocks
//      and publishes them as tagged entries (the launch's tag in the high
//      word, so an entry is its own ready flag);
//   2. attention items, one per (unit, split), unit-major: each wave waits
//      (bounded spin, never expected to be long) until its entries carry the
//      launch's tag, then attends.
// Scoring never waits and every scoring item precedes every attention item,
// so the waits always end.  By the time the attention items of the last units
// are reached, their selections have run behind the attention of earlier units,
// so selection latency is mostly off the critical path.  The device functions
// are the same as the stand-alone kernels', so results are identical to the
// three calls.
//
// The launch tag is one more than a launch counter kept in the queue words; the
// last workgroup to leave advances the counter (skipping the value whose
// successor would be 0, so that a tag is never 0 and two launches in a row never
// share one) and re-arms the queue.
#include "attend_dev.h"
#include "select_dev.h"

namespace btk {
namespace {

using sel::kMaxChunk;
using sel::kThreads;
using sel::kWaves;

struct StepArgs {
    sel::SelectArgs s;
    att::AttendArgs t;
    uint64_t *tagged;  // [units][top_k] published selections (also t.tagged)
    uint32_t *queue;   // [0] items taken beyond the grid, [1] workgroups that have left,
                       // [2] launch counter
    int B, units, nsplit;
};

constexpr int kStageBlocks = 1;  // bf16 attention pipeline stage (fp32: 2, see attend.hip)
constexpr int kScanRows = 4;     // centroid rows per lane per scan stage

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void decode_step_kernel(StepArgs a) {
    __shared__ float qs[D];
    __shared__ int pages[kMaxChunk];
    __shared__ float sc_lds[kMaxChunk];
    __shared__ int flag;
    __shared__ uint32_t hist[256 + kWave], cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ float crow[kWaves * D];
    __shared__ uint32_t prefix[kMaxStepBatch + 1];  // scoring items before each sequence
    __shared__ int item_s;
    __shared__ uint32_t tag_s;
    // queries while scoring, top-k keys of long contexts, attention merges
    extern __shared__ float dyn[];
    sel::ScoreSmem sm{dyn, qs, pages, sc_lds, &flag};
    sel::TopkSmem tk{hist, cand, red, scan_red, reinterpret_cast<uint32_t *>(dyn)};
    const int tid = threadIdx.x;
    const int Hkv = a.s.Hkv;

    // the launch tag is fetched while the prefix is built; the first item is
    // the workgroup's own index, later ones come from the queue (offset by the
    // grid), so the launch does not open with every workgroup's atomic at once
    if (tid == 0)
        tag_s = __hip_atomic_load(&a.queue[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    // scoring items per sequence: Hkv * chunks (one item for an invalid length,
    // which writes -1 indices and flags the error)
    for (int b0 = 0; b0 < a.B; b0 += kThreads) {
        const int b = b0 + tid;
        uint32_t n = 0;
        if (b < a.B) {
            const int L = a.s.seq_lens[b];
            const bool ok = L >= 1 && L <= a.s.max_blocks * kPage;
            const int nb = ok ? (L + kPage - 1) / kPage : 0;
            n = (uint32_t)Hkv * (uint32_t)(ok ? (nb + a.s.chunk - 1) / a.s.chunk : 1);
        }
        const uint32_t carry = b0 == 0 ? 0u : prefix[b0];
        const int before = sel::wg_exclusive_scan((int)n, scan_red);
        if (b < a.B) prefix[b + 1] = carry + (uint32_t)before + n;
        if (b0 == 0 && tid == 0) prefix[0] = 0u;
        __syncthreads();
    }
    const int n_score = (int)prefix[a.B];
    const int total = n_score + a.units * a.nsplit;

    const uint32_t tag = tag_s;
    int item = (int)blockIdx.x;
    // the next item from the queue (LDS is reused by the next item)
    auto next_item = [&]() {
        __syncthreads();
        if (tid == 0) item_s = (int)(gridDim.x + atomicAdd(&a.queue[0], 1u));
        __syncthreads();
        return item_s;
    };
    // every scoring item precedes every attention item, so a workgroup runs
    // the two kinds in two loops (each with registers of its own)
    int b_cur = 0;
    while (item < n_score) {
        while ((int)prefix[b_cur + 1] <= item) ++b_cur;  // items only grow
        const int nc = (int)(prefix[b_cur + 1] - prefix[b_cur]) / Hkv;
        const int rel = item - (int)prefix[b_cur];
        // a unit's chunks go last to first: the one that refreshes the newest
        // page starts first, so that it is rarely the one left to select
        const int unit = b_cur * Hkv + rel / nc, c = nc - 1 - rel % nc;
        int nb = 0;
        if (sel::score_chunk<T, D, kScanRows>(a.s, unit, c, sm, crow, nb)) {
            __builtin_amdgcn_s_setprio(3);
            sel::select_topk(sel::PlainScores{a.s.scores + (size_t)unit * a.s.max_blocks},
                             nb, a.s.top_k,
                             sel::TopkOut{a.s.indices + (size_t)unit * a.s.top_k,
                                          a.tagged + (size_t)unit * a.s.top_k, tag},
                             tk);
            __builtin_amdgcn_s_setprio(0);
        }
        item = next_item();
    }
    while (item < total) {
        const int rel = item - n_score;
        att::attend_item<T, D, att::kSelected, (sizeof(T) == 4 ? 2 : kStageBlocks)>(
            a.t, rel / a.nsplit, rel % a.nsplit, dyn, &flag, tag);
        item = next_item();
    }
    // the last workgroup to leave re-arms the queue and advances the counter
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&a.queue[1], 1u);
        if (prev == gridDim.x - 1) {
            __hip_atomic_store(&a.queue[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.queue[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.queue[2], tag == 0xffffffffu ? 0u : tag, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t step_lds_floats(const Dims &d, const AttendPlan &ap) {
    const size_t r = d.group();
    size_t n = r * d.D;                                              // queries
    const size_t wave_merge = (size_t)att::kWaves * r * d.D + 2 * att::kWaves * 16;
    const size_t split_merge = 2 * (size_t)ap.nsplit_max * r + r;
    n = n > wave_merge ? n : wave_merge;
    n = n > split_merge ? n : split_merge;
    if (d.max_blocks > 32 * kWave && (size_t)d.max_blocks > n) n = d.max_blocks;  // top-k keys
    return n;
}

// resident workgroups of the step kernel on this device (cached per device)
template <typename T, int D>
hipError_t resident_workgroups(size_t lds, int *out) {
    static int cached[64][2] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int slot = dev & 63;
    if (cached[slot][0] > 0 && cached[slot][1] == (int)lds) {
        *out = cached[slot][0];
        return hipSuccess;
    }
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_step_kernel<T, D>, kThreads,
                                                     lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[slot][0] = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    cached[slot][1] = (int)lds;
    *out = cached[slot][0];
    return hipSuccess;
}

template <typename T, int D>
hipError_t launch(const Dims &d, const SelectPlan &sp, const AttendPlan &ap, StepArgs a,
                  hipStream_t stream) {
    const size_t lds = sizeof(float) * step_lds_floats(d, ap);
    int grid = 0;
    hipError_t e = resident_workgroups<T, D>(lds, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_step_kernel<T, D>), dim3(grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(const Dims &d, const SelectPlan &sp, const AttendPlan &ap,
                              const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *first_pos, float *centroids, int top_k,
                              int32_t *indices, float *scores, void *out, float *lse,
                              float *partials, uint32_t *sel_counters, uint32_t *att_counters,
                              uint64_t *tagged, uint32_t *queue, uint32_t *err,
                              hipStream_t stream) {
    StepArgs a;
    a.s = sel::SelectArgs{q, centroids, block_table, seq_lens, indices, scores, sel_counters, err,
                          d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, sp.chunk, sp.nchunk_max,
                          d.sm_scale, k_cache, first_pos, centroids};
    a.t = att::AttendArgs{q, k_cache, v_cache, block_table, seq_lens, indices, out, lse, partials,
                          att_counters, err, d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, ap.bps,
                          ap.nsplit_max, d.sm_scale * 1.44269504088896340736f, tagged, nullptr};
    a.tagged = tagged;
    a.queue = queue;
    a.B = d.B;
    a.units = d.B * d.Hkv;
    a.nsplit = ap.nsplit_max;
    if (d.dtype == 0)
        return d.D == 128 ? launch<uint16_t, 128>(d, sp, ap, a, stream)
                          : launch<uint16_t, 64>(d, sp, ap, a, stream);
    return d.D == 128 ? launch<float, 128>(d, sp, ap, a, stream)
                      : launch<float, 64>(d, sp, ap, a, stream);
}

}  // namespace btk
