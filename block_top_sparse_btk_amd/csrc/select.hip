// S2 + S3 stand-alone: group block scoring and top-k selection in one launch
// (device code in select_dev.h).  Grid = units x chunks; the workgroup that
// finishes a unit's last chunk selects its top-k blocks.  The shared-prefix
// form adds, ahead of them, items that score each group's shared prefix once
// (shared_item); the members' own chunks then cover their private blocks.
#include "select_dev.h"

namespace btk {
using namespace sel;
namespace {

// Shared-prefix scoring (Best-of-N): a workgroup per (group, KV head, chunk of
// the shared prefix) reads each shared centroid row once and scores it against
// every member's mean query, with the same arithmetic as score_chunk, so the
// scores are bit-identical to scoring every member alone; it checks that every
// member's table slice equals the first member's.  Once its stores are done it
// counts itself in on the (group, KV head) flag; the members' own chunks
// complete and select for them (see select_kernel), so the selections of a
// group run in parallel.
template <typename T, int D>
__device__ __forceinline__ void shared_item(const SelectArgs &a, const PrefixGroups &pg, int item,
                                            float *qs, int *pages, int *flags) {
    constexpr int LPR = 16, VPL = D / LPR, RPI = kWave / LPR;
    constexpr int KU = kSharedChunk / (kWaves * RPI);  // one stage covers an item
    constexpr int ROWS = kWaves * RPI * KU;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int g = 0;
    while (g + 1 < pg.n && pg.item0[g + 1] <= item) ++g;
    const int P = pg.blocks[g], first = pg.start[g], M = pg.start[g + 1] - first;
    const int ncs = (P + kSharedChunk - 1) / kSharedChunk;
    const int rel = item - pg.item0[g], gk = rel / ncs, c = rel % ncs;
    const int j0 = c * kSharedChunk, n = min(P, j0 + kSharedChunk) - j0;
    const int r = a.Hq / a.Hkv;

    // set-up in one round trip: the first member's page ids, every member's
    // queries (summed in head order, as score_chunk does) and length
    if (tid < M) flags[tid] = 0;
    for (int i = tid; i < n; i += kThreads) {
        int p = a.bt[(size_t)first * a.max_blocks + j0 + i];
        if (p < 0 || p >= a.num_pages) {
            flag_error(a.err, kErrPage);
            p = -1;
        }
        pages[i] = p;
    }
    // the (member, dim) pairs of this thread, QB at a time; the loads are
    // unconditional (clamped to valid addresses, values masked after) so that
    // they are all in flight together rather than one branch at a time; heads
    // are summed in order, as score_chunk does
    constexpr int QB = 4, HB = 8;
    for (int i0 = tid; i0 < M * D; i0 += QB * kThreads) {
        float s[QB] = {};
        for (int h0 = 0; h0 < r; h0 += HB) {
            float x[QB][HB];
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int idx = min(i0 + u * kThreads, M * D - 1);
                const int m = idx / D, dd = idx % D;
                const T *qp = static_cast<const T *>(a.q) +
                              ((size_t)(first + m) * a.Hq + (size_t)gk * r) * D + dd;
#pragma unroll
                for (int h = 0; h < HB; ++h) x[u][h] = load_q<T>(qp + min(h0 + h, r - 1) * D);
            }
#pragma unroll
            for (int u = 0; u < QB; ++u)
                for (int h = 0; h < HB && h0 + h < r; ++h) s[u] += x[u][h];
        }
#pragma unroll
        for (int u = 0; u < QB; ++u)
            if (i0 + u * kThreads < M * D) qs[i0 + u * kThreads] = s[u] * (a.scale / (float)r);
    }
    __syncthreads();
    {  // every member's slice against the first member's (loads in flight together)
        constexpr int kV = 8;
        for (int i0 = tid; i0 < (M - 1) * n; i0 += kThreads * kV) {
            int x[kV], y[kV];
#pragma unroll
            for (int u = 0; u < kV; ++u) {
                const int i = min(i0 + u * kThreads, (M - 1) * n - 1);
                const int m = 1 + i / n, j = i % n;
                x[u] = a.bt[(size_t)(first + m) * a.max_blocks + j0 + j];
                y[u] = pages[j];
            }
#pragma unroll
            for (int u = 0; u < kV; ++u)
                if (x[u] != y[u] && y[u] >= 0) flags[kMaxGroupMembers] = 1;
        }
    }

    const int col = lane % LPR, rsub = lane / LPR;
    typedef floatx4_t Row[VPL / 4];
    auto issue = [&](Row (&cv)[KU], int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = min(base + u * kWaves * RPI + wave * RPI + rsub, n - 1);
            const int p = max(pages[row], 0);
            const floatx4_t *src = reinterpret_cast<const floatx4_t *>(
                a.cent + ((size_t)p * a.Hkv + gk) * D + col * VPL);
#pragma unroll
            for (int v = 0; v < VPL / 4; ++v) cv[u][v] = src[v];
        }
    };
    auto reduce = [&](const Row (&cv)[KU], int base) {
        for (int m = 0; m < M; ++m) {
            float qf[VPL];
#pragma unroll
            for (int e = 0; e < VPL; ++e) qf[e] = qs[m * D + col * VPL + e];
            float *sc = a.scores + ((size_t)(first + m) * a.Hkv + gk) * a.max_blocks + j0;
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int row = base + u * kWaves * RPI + wave * RPI + rsub;
                const float s = row16_sum(row_partial<VPL>(qf, cv[u]));
                if (col == 0 && row < n) store_relaxed(sc + row, pages[row] >= 0 ? s : -INFINITY);
            }
        }
    };
    if (n > 0) {
        Row ca[KU], cb[KU];
        issue(ca, 0);
        for (int base = 0;;) {
            issue(cb, base + ROWS);
            reduce(ca, base);
            base += ROWS;
            if (base >= n) break;
            issue(ca, base + ROWS);
            reduce(cb, base);
            base += ROWS;
            if (base >= n) break;
        }
    }

    // count in on the (group, KV head) flag once the scores are stored
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        if (flags[kMaxGroupMembers]) flag_error(a.err, kErrPrefix);
        __hip_atomic_fetch_add(&a.pflags[((size_t)g * a.Hkv + gk) * kStateStride], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <typename T, int D, bool SHARED>
__global__ __launch_bounds__(kThreads, SHARED ? 4 : 5) void select_kernel(SelectArgs a, PrefixGroups pg) {
    __shared__ float qraw[(SHARED ? kMaxGroupMembers : kMaxGroup) * D];
    __shared__ float qs[D];
    __shared__ int pages[kMaxChunk];
    __shared__ float sc_lds[kMaxChunk];
    __shared__ int is_last;
    // read as 16-byte vectors (histogram bins, candidate keys): 16-byte aligned
    __shared__ __align__(16) uint32_t hist[sel::kTopkPasses * sel::kHistWords];
    __shared__ __align__(16) uint32_t cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ int flags[SHARED ? kMaxGroupMembers + 1 : 1];
    extern __shared__ uint32_t keys[];  // 512 words: top-k bitmaps beyond 2048 blocks
    ScoreSmem sm{qraw, qs, pages, sc_lds, &is_last};
    TopkSmem tk{hist, cand, red, scan_red, keys};
    int item = blockIdx.x;
    int skip = 0;  // a shared prefix, scored by shared items
    int grp = -1;  // the group of this item's sequence
    if (SHARED) {
        if (item < pg.item0[pg.n]) {  // the shared items come first and never wait
            if (threadIdx.x <= kMaxGroupMembers) flags[threadIdx.x] = 0;
            __syncthreads();
            shared_item<T, D>(a, pg, item, qraw, pages, flags);
            return;
        }
        item -= pg.item0[pg.n];
        const int b = item / a.nchunk_max / a.Hkv;
        for (int g = 0; g < pg.n; ++g)
            if (pg.start[g] <= b && b < pg.start[g + 1]) {
                skip = pg.blocks[g];
                grp = g;
            }
    }
    const int unit = item / a.nchunk_max, c = item % a.nchunk_max;
    int nb = 0;
    const bool completes = score_chunk<T, D, 4>(a, unit, c, sm, nullptr, nb, skip, 0);
    // a group member that completed (or, with an invalid length, its only item)
    // waits until the group's shared items of its KV head are done, and counts
    // out afterwards; the last member to count out clears the flag
    const bool member = SHARED && grp >= 0 && (completes || (nb < 0 && c == 0));
    uint32_t *pf = member ? a.pflags + ((size_t)grp * a.Hkv + unit % a.Hkv) * kStateStride : nullptr;
    if (member) {
        const uint32_t shared_items =
            (uint32_t)((pg.item0[grp + 1] - pg.item0[grp]) / a.Hkv);
        if (threadIdx.x == 0) {
            for (uint32_t spins = 0;
                 __hip_atomic_load(pf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < shared_items;
                 ++spins) {
                if (spins > (1u << 22)) {  // never expected: report, do not hang
                    flag_error(a.err, kErrTimeout);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
    }
    if (completes) {
        // the selecting wave(s) take issue priority over scanning waves on the SIMD
        __builtin_amdgcn_s_setprio(3);
        select_topk(PlainScores{a.scores + (size_t)unit * a.max_blocks}, nb, a.top_k,
                    TopkOut{a.indices + (size_t)unit * a.top_k}, tk);
        __builtin_amdgcn_s_setprio(0);
    }
    if (member && threadIdx.x == 0) {
        const uint32_t members = (uint32_t)(pg.start[grp + 1] - pg.start[grp]);
        const uint32_t prev =
            __hip_atomic_fetch_add(pf + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1 == members) {
            __hip_atomic_store(pf, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pf + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Compute units of the current device (cached per device).
hipError_t device_cus(int *out) {
    static int cached[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int &c = cached[dev & 63];
    if (c <= 0) {
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (c <= 0) c = 1;
    }
    *out = c;
    return hipSuccess;
}

// The chunk: the smallest multiple of 64 blocks from 128 up whose chunks all fit
// in one round of resident workgroups (five per CU by the kernel's launch
// bounds, four in the shared-prefix form, whose shared items come first) even
// if every sequence had max_blocks blocks.  Smaller chunks shorten the tail in
// which only the largest chunks are still streaming; chunks that wait for a
// free slot lengthen it more.  Measured on the Qwen3-8B-shaped batch: chunks of
// 512 blocks 40.2 us, 448 37.5 us (this rule), 256 44.4 us (about as many
// chunks as slots); the other workloads within 1 us of their best size.
SelectPlan fit_chunks(const Dims &d, int cus, int per_cu, int extra) {
    const size_t units = (size_t)d.B * d.Hkv;
    const size_t slots = (size_t)cus * per_cu;
    int chunk = 128;
    while (chunk < kMaxChunk &&
           units * (size_t)((d.max_blocks + chunk - 1) / chunk) + (size_t)extra > slots)
        chunk += 64;
    SelectPlan p;
    p.chunk = chunk;
    p.nchunk_max = (d.max_blocks + chunk - 1) / chunk;
    return p;
}

template <typename T, int D>
hipError_t launch(const Dims &d, const SelectPlan &, SelectArgs a, const PrefixGroups *pg,
                  hipStream_t stream) {
    int cus = 0;
    const hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const SelectPlan plan = fit_chunks(d, cus, pg ? 4 : 5, pg ? pg->item0[pg->n] : 0);
    a.chunk = plan.chunk;
    a.nchunk_max = plan.nchunk_max;
    const size_t grid = (size_t)d.B * d.Hkv * plan.nchunk_max;
    // the top-k bitmaps of more than 2048 blocks (two words per 32 blocks)
    const size_t lds = d.max_blocks > 32 * kWave ? sizeof(uint32_t) * 512 : 0;
    if (pg)
        hipLaunchKernelGGL((select_kernel<T, D, true>), dim3((unsigned)(grid + pg->item0[pg->n])),
                           dim3(kThreads), lds, stream, a, *pg);
    else
        hipLaunchKernelGGL((select_kernel<T, D, false>), dim3((unsigned)grid), dim3(kThreads),
                           lds, stream, a, PrefixGroups{});
    return hipGetLastError();
}

}  // namespace

SelectPlan plan_select(const Dims &d) {
    // (host default without a device query; the select launch refits the chunk
    // to the device, see fit_chunks)
    // At least about 1024 chunks, each as large as that allows.
    const size_t rows = (size_t)d.B * d.Hkv * d.max_blocks;
    int chunk = 64;
    while (chunk < kMaxChunk && rows / (size_t)(chunk * 2) >= 1024) chunk *= 2;
    SelectPlan p;
    p.chunk = chunk;
    p.nchunk_max = (d.max_blocks + chunk - 1) / chunk;
    return p;
}

hipError_t launch_select(const Dims &d, const SelectPlan &plan, const void *q,
                         const float *centroids, const int32_t *block_table,
                         const int32_t *seq_lens, int top_k, int32_t *indices, float *scores,
                         uint32_t *counters, uint32_t *err, hipStream_t stream) {
    SelectArgs a{q, centroids, block_table, seq_lens, indices, scores, counters, err,
                 d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, plan.chunk, plan.nchunk_max,
                 d.sm_scale, nullptr, nullptr, nullptr};
    if (d.dtype == 0)
        return d.D == 128 ? launch<uint16_t, 128>(d, plan, a, nullptr, stream)
                          : launch<uint16_t, 64>(d, plan, a, nullptr, stream);
    return d.D == 128 ? launch<float, 128>(d, plan, a, nullptr, stream)
                      : launch<float, 64>(d, plan, a, nullptr, stream);
}

hipError_t launch_select_shared(const Dims &d, const SelectPlan &plan, const PrefixGroups &pg,
                                const void *q, const float *centroids,
                                const int32_t *block_table, const int32_t *seq_lens, int top_k,
                                int32_t *indices, float *scores, uint32_t *counters,
                                uint32_t *pflags, uint32_t *err, hipStream_t stream) {
    SelectArgs a{q, centroids, block_table, seq_lens, indices, scores, counters, err,
                 d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, plan.chunk, plan.nchunk_max,
                 d.sm_scale, nullptr, nullptr, nullptr, pflags};
    if (d.dtype == 0)
        return d.D == 128 ? launch<uint16_t, 128>(d, plan, a, &pg, stream)
                          : launch<uint16_t, 64>(d, plan, a, &pg, stream);
    return d.D == 128 ? launch<float, 128>(d, plan, a, &pg, stream)
                      : launch<float, 64>(d, plan, a, &pg, stream);
}

}  // namespace btk
