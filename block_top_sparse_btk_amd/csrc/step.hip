// Single-launch decode step: S1 (touched pages) + S2 + S3 + S4 in one persistent
// kernel.  (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What
// carries the argument": averaged-key block summaries, per-query-group scoring,
// top-k blocks, attention over the kept blocks.)
//
// Phase 1, scoring.  The launch's centroid rows, ordered by sequence, KV head
// and block (each unit charged kSegmentCost extra rows for its fixed costs), are
// cut as follows: the first 7/8 into one equal, contiguous share per
// workgroup, the rest into chunks that the workgroups finishing first take
// from a counter, so that the scan ends at about the same time everywhere.  A
// share or chunk is a few segments (a run of one unit's blocks, a unit usually
// spanning two or three workgroups), each scored in runs of up to kRun blocks;
// the run that holds a touched page first recomputes its centroid (S1).  A
// segment then adds its block count to the unit's counter, and the segment that
// completes the unit marks it ready with the launch's tag.
//
// Phase 2, selection and attention.  Item (unit, split) i is taken by
// workgroup i mod G.  It waits (bounded spin, never expected to be long) until
// its unit is ready, selects the unit's top-k blocks from the stored scores
// (S3), keeps its split's share of the selection in LDS and attends (S4).  Each
// split of a unit selects for itself (identical results), split 0 also writes
// the indices.  Scoring never waits and a workgroup ends its scoring (share and
// chunks, until none is left) before it takes an item, so every wait ends.
//
// Handing out all scoring work in dynamic chunks was measured slower: the last
// chunks to be handed out run at a fair share of the bandwidth next to the
// attention of earlier units and set the end of the launch.
//
// The launch tag is one more than a launch counter kept in the queue words; the
// last workgroup to leave advances the counter (skipping the value whose
// successor would be 0, so that a tag is never 0 and two launches in a row never
// share one) and re-arms the chunk counter and the queue words.
#include "attend_dev.h"
#include "select_dev.h"

namespace btk {
namespace {

using sel::kThreads;
using sel::kWaves;

struct StepArgs {
    sel::SelectArgs s;
    att::AttendArgs t;
    uint32_t *ready;  // [units * kReadyStride]: word u * kReadyStride is unit u's ready tag
    uint32_t *queue;  // [0] spare, [1] workgroups that have left, [2] launch counter
    uint32_t *steal;  // scan chunks taken (a line of its own)
    int B, units, nsplit;
};

constexpr int kStageBlocks = 1;  // bf16 attention pipeline stage (fp32: 2, see attend.hip)
constexpr int kScanRows = 4;     // centroid rows per lane per scan stage
constexpr int kRun = 2048;       // blocks per scan run: shares (~550 blocks at 32 x 8 units of
                                 // 17K tokens) take one run, one page-id round trip; in phase 2
                                 // the page-id area holds the block-table row of units of up to
                                 // kRun blocks
// Rows charged for a unit beyond its blocks when the shares are cut: a segment
// costs round trips in which nothing streams (its setup, its closing
// store-and-count) and the unit's touched page its refresh, so a share that
// starts a unit gets that many fewer blocks.  The charge also moves share ends
// earlier for the workgroups that start units, which then take more of the
// stolen chunks.  Measured on the Qwen3-8B-shaped step (three length draws) and
// on uniform-length batches of 64 to 512 units: 160 -> 520 rows shortened the
// ragged steps by 1.4-2.8 us and left the others equal or faster; from about
// 700 rows on the ragged steps got slower again.
constexpr int kSegmentCost = 520;
// The last 1/kStealFrac of the rows is handed out in chunks of kStealRows to the
// workgroups that finish their static share first.
constexpr int kStealFrac = 8;
constexpr uint32_t kStealRows = 256;

// KV append (APPEND): the newest token of unit (b, g), position L - 1, goes
// into slot (L - 1) % 16 of its page in both caches.  Phase 1 takes its key
// from k_new for the block's centroid and never reads that slot; the unit's
// attention item writes the slot (each split of the unit the same values) while
// its ready poll and selection run, and waits for its own stores before it
// attends, so no other workgroup reads the slot in this launch.  The value cache
// is dim-major: the slot is one element per dimension.
template <typename T, int D>
__device__ __forceinline__ void append_to_cache(const StepArgs &a, int b, int g, int L,
                                                int lane) {
    constexpr int W = D * (int)sizeof(T) / 4;  // 32-bit words per row
    const int jn = (L - 1) / kPage, t = (L - 1) % kPage;
    const int page = a.s.bt[(size_t)b * a.s.max_blocks + jn];
    const size_t row = ((size_t)b * a.s.Hkv + g) * D;
    uint32_t kw[(W + kWave - 1) / kWave];
    T vv[(D + kWave - 1) / kWave];
#pragma unroll
    for (int i = 0; i < (W + kWave - 1) / kWave; ++i)
        kw[i] = reinterpret_cast<const uint32_t *>(static_cast<const T *>(a.s.k_new) + row)
            [min(lane + i * kWave, W - 1)];
#pragma unroll
    for (int i = 0; i < (D + kWave - 1) / kWave; ++i)
        vv[i] = static_cast<const T *>(a.s.v_new)[row + min(lane + i * kWave, D - 1)];
    if (page < 0 || page >= a.s.num_pages) return;  // flagged by the scan of that block
    const size_t tile = ((size_t)page * a.s.Hkv + g) * kPage * D;
    uint32_t *kd = reinterpret_cast<uint32_t *>(static_cast<T *>(a.s.k_out) + tile + (size_t)t * D);
#pragma unroll
    for (int i = 0; i < (W + kWave - 1) / kWave; ++i)
        if (lane + i * kWave < W) kd[lane + i * kWave] = kw[i];
    T *vd = static_cast<T *>(a.s.v_out) + tile + t;
#pragma unroll
    for (int i = 0; i < (D + kWave - 1) / kWave; ++i)
        if (lane + i * kWave < D) vd[(size_t)(lane + i * kWave) * kPage] = vv[i];
}

// APPEND: the KV append of the step is fused in (a separate instantiation, so
// that the plain step carries none of its code).
template <typename T, int D, bool APPEND>
__global__ __launch_bounds__(kThreads, 2) void decode_step_kernel(StepArgs a) {
    __shared__ float qs[D];
    __shared__ int pages[kRun];
    __shared__ float sc_lds[kRun];
    __shared__ int flag;
    __shared__ uint32_t hist[sel::kTopkPasses * sel::kHistWords], cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ float crow[kWaves * D];
    __shared__ __align__(16) uint32_t newtok[APPEND ? D * sizeof(T) / 4 : 4];  // new key
    __shared__ uint32_t rows[kMaxStepBatch + 1];  // centroid rows before each sequence
    __shared__ int lens[kMaxStepBatch];           // sequence lengths, -1: invalid
    __shared__ int fps[kMaxStepBatch];            // decode positions (first touched token)
    __shared__ int item_s;
    __shared__ uint32_t tag_s;
    // queries while scoring, top-k keys of long contexts, attention merges
    extern __shared__ float dyn[];
    sel::ScoreSmem sm{dyn, qs, pages, sc_lds, &flag, newtok};
    sel::TopkSmem tk{hist, cand, red, scan_red, reinterpret_cast<uint32_t *>(dyn)};
    const int tid = threadIdx.x;
    const int Hkv = a.s.Hkv;

    // the launch tag is fetched while the row prefix is built: per unit
    // kSegmentCost charged rows, then one row per block (a single placeholder
    // row for an invalid length, which writes -1 indices and flags the error)
    if (tid == 0)
        tag_s = __hip_atomic_load(&a.queue[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    for (int b0 = 0; b0 < a.B; b0 += kThreads) {
        const int b = b0 + tid;
        uint32_t n = 0;
        if (b < a.B) {
            const int L = a.s.seq_lens[b];
            const bool ok = L >= 1 && L <= a.s.max_blocks * kPage;
            const int nb = ok ? (L + kPage - 1) / kPage : -1;
            lens[b] = ok ? L : -1;
            // with the KV append the newest token (L - 1) is the one touched
            fps[b] = APPEND ? (ok ? L - 1 : -1) : a.s.first_pos ? a.s.first_pos[b] : -1;
            n = (uint32_t)Hkv * (uint32_t)(kSegmentCost + (ok ? nb : 1));
        }
        const uint32_t carry = b0 == 0 ? 0u : rows[b0];
        const int before = sel::wg_exclusive_scan((int)n, scan_red);
        if (b < a.B) rows[b + 1] = carry + (uint32_t)before + n;
        if (b0 == 0 && tid == 0) rows[0] = 0u;
        __syncthreads();
    }
    const uint32_t tag = tag_s;

    // ---- phase 1: this workgroup's static share of the first rows, then chunks
    // of the rest while any are left (shares end at different times: the
    // workgroups that finish first take more of the rest)
    const uint64_t R = rows[a.B];
    const uint64_t RS = R - R / kStealFrac;
    uint32_t r = (uint32_t)(RS * blockIdx.x / gridDim.x);
    uint32_t r1 = (uint32_t)(RS * (blockIdx.x + 1) / gridDim.x);
    int b = 0;
    for (;;) {
        if (r >= r1) {
            if (tid == 0) item_s = (int)atomicAdd(a.steal, 1u);
            __syncthreads();
            const uint64_t c0 = RS + (uint64_t)item_s * kStealRows;
            __syncthreads();  // item_s is written again
            if (c0 >= R) break;
            r = (uint32_t)c0;
            r1 = (uint32_t)min(R, c0 + kStealRows);
        }
        while (rows[b + 1] <= r) ++b;
        const int nb = lens[b] < 0 ? -1 : (lens[b] + kPage - 1) / kPage;
        const uint32_t per_unit = kSegmentCost + (nb < 0 ? 1u : (uint32_t)nb);
        const uint32_t off = r - rows[b];
        const uint32_t g = off / per_unit, o = off % per_unit;  // o < kSegmentCost: charged rows
        const uint32_t e = min(per_unit, o + (r1 - r));         // this share's end in the unit
        const int j0 = (int)(o > kSegmentCost ? o - kSegmentCost : 0u);
        const int j1 = (int)(e > kSegmentCost ? e - kSegmentCost : 0u);
        if (j1 > j0) {
            sel::score_segment<T, D, kScanRows, kRun, APPEND>(
                a.s, b, (int)g, j0, j1, nb, lens[b], fps[b], sm, crow,
                a.ready + ((size_t)b * Hkv + g) * kReadyStride, tag);
            __syncthreads();  // LDS is reused by the next segment
        }
        r += e - o;
    }

    // ---- phase 2: (unit, split) items
    const int total = a.units * a.nsplit;
    int32_t *list = reinterpret_cast<int32_t *>(sc_lds);  // the split's share, <= 256 entries
    // item i goes to workgroup i mod G: with fewer items than resident
    // workgroups the first G/2 take one each, one per CU (workgroups are
    // placed on CUs in index order), so no CU runs two attentions at once
    for (int item = (int)blockIdx.x;; item += (int)gridDim.x) {
        __syncthreads();  // LDS is reused
        if (item >= total) break;
        const int unit = item / a.nsplit, split = item % a.nsplit;
        const int bu = unit / Hkv;
        const int L = lens[bu];
        const int nb = L < 0 ? -1 : (L + kPage - 1) / kPage;
        // the sequence's block-table row is requested before the wait, so that
        // the attention finds the selected blocks' pages in LDS
        const bool row_lds = nb >= 0 && nb <= kRun;
        constexpr int kRowPer = kRun / kThreads;
        int32_t prow[kRowPer];
        if (row_lds) {
            const int32_t *bt_row = a.s.bt + (size_t)bu * a.s.max_blocks;
#pragma unroll
            for (int i = 0; i < kRowPer; ++i)  // unconditional: all in flight together
                prow[i] = bt_row[min(i * kThreads + tid, nb - 1)];
        }
        if (APPEND && nb >= 0 && tid >= kWave && tid < 2 * kWave)  // wave 1, beside the poll
            append_to_cache<T, D>(a, bu, unit % Hkv, L, tid - kWave);
        if (tid == 0) {
            const uint32_t *rw = a.ready + (size_t)unit * kReadyStride;
            uint32_t spins = 0;
            while (__hip_atomic_load(rw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) {
                if (++spins > att::kReadySpinLimit) {  // never expected: report, do not hang
                    flag_error(a.s.err, kErrTimeout);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
        const int lo = split * a.t.bps, hi = min(a.s.top_k, lo + a.t.bps);
        if (nb >= 0) {
            __builtin_amdgcn_s_setprio(3);
            sel::select_topk(sel::PlainScores{a.s.scores + (size_t)unit * a.s.max_blocks}, nb,
                             a.s.top_k,
                             sel::TopkOut{split == 0 ? a.s.indices + (size_t)unit * a.s.top_k
                                                     : nullptr,
                                          list, lo, hi},
                             tk);
            __builtin_amdgcn_s_setprio(0);
        }
        if (row_lds) {
#pragma unroll
            for (int i = 0; i < kRowPer; ++i)
                if (i * kThreads + tid < nb) pages[i * kThreads + tid] = prow[i];
        }
        // the appended token's cache stores are done before the block can be read
        if (APPEND) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        att::attend_item<T, D, att::kSelected, (sizeof(T) == 4 ? 2 : kStageBlocks)>(
            a.t, unit, split, dyn, &flag, list, L < 0 ? 0 : L, row_lds ? pages : nullptr);
        __syncthreads();  // LDS is reused by the next item
    }
    // the last workgroup to leave re-arms the queue and advances the counter
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&a.queue[1], 1u);
        if (prev == gridDim.x - 1) {
            __hip_atomic_store(&a.queue[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.steal, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
template <typename T, int D, bool APPEND>
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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_step_kernel<T, D, APPEND>,
                                                     kThreads, lds);
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
    hipError_t e;
    if (a.s.k_new) {
        e = resident_workgroups<T, D, true>(lds, &grid);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((decode_step_kernel<T, D, true>), dim3(grid), dim3(kThreads), lds,
                           stream, a);
    } else {
        e = resident_workgroups<T, D, false>(lds, &grid);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((decode_step_kernel<T, D, false>), dim3(grid), dim3(kThreads), lds,
                           stream, a);
    }
    return hipGetLastError();
}

}  // namespace

bool step_rows_fit(const Dims &d) {
    return (uint64_t)d.B * (uint64_t)d.Hkv * ((uint64_t)d.max_blocks + kSegmentCost) <
           ((uint64_t)1 << 32);
}

hipError_t launch_decode_step(const Dims &d, const SelectPlan &sp, const AttendPlan &ap,
                              const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *first_pos, float *centroids, int top_k,
                              int32_t *indices, float *scores, void *out, float *lse,
                              float *partials, uint32_t *sel_counters, uint32_t *att_counters,
                              uint32_t *ready, uint32_t *queue, uint32_t *steal,
                              uint32_t *err, hipStream_t stream, const void *k_new,
                              const void *v_new) {
    // a split's share of the selection (at most 4 * 64 entries) is kept in the
    // score staging area
    if (ap.bps > kRun) return hipErrorInvalidValue;
    StepArgs a;
    a.s = sel::SelectArgs{q, centroids, block_table, seq_lens, indices, scores, sel_counters, err,
                          d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, sp.chunk, sp.nchunk_max,
                          d.sm_scale, k_cache, first_pos, centroids};
    if (k_new) {  // the caches are the caller's, written in place by the append
        a.s.k_new = k_new;
        a.s.v_new = v_new;
        a.s.k_out = const_cast<void *>(k_cache);
        a.s.v_out = const_cast<void *>(v_cache);
        a.s.first_pos = nullptr;
    }
    a.t = att::AttendArgs{q, k_cache, v_cache, block_table, seq_lens, indices, out, lse, partials,
                          att_counters, err, d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, ap.bps,
                          ap.nsplit_max, d.sm_scale * 1.44269504088896340736f, nullptr};
    a.ready = ready;
    a.queue = queue;
    a.steal = steal;
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
