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
// Every share is claimed before it is scored (one atomic per share, issued with
// the prologue's loads, so its round trip costs nothing): by its own workgroup
// when that one starts, or else by workgroup 0 or a workgroup that holds no
// phase-2 item, which look for unclaimed shares once their own scoring is done.
// Workgroup 0 is dispatched before any other, so every share is claimed by a
// running workgroup, and every slice of the scan is done without waiting: a
// phase-2 wait therefore always ends, whether or not the whole grid is
// resident (another kernel may hold part of the device).
//
// Phase 2, selection and attention.  Item (unit, split) i is taken by
// workgroup i mod G.  It waits (bounded spin, as a safeguard only) until its
// unit is ready, selects the unit's top-k blocks from the stored scores (S3),
// keeps its split's share of the selection in LDS and attends (S4).  Each split
// of a unit selects for itself (identical results), split 0 also writes the
// indices.
//
// Handing out all scoring work in dynamic chunks was measured slower: the last
// chunks to be handed out run at a fair share of the bandwidth next to the
// attention of earlier units and set the end of the launch.  So was claiming
// the shares in small slices that idle workgroups could take from slow ones
// (every claim and every extra segment is a round trip, several microseconds
// while the scan saturates the memory system).
//
// The launch tag is one more than a launch counter kept in the queue words; the
// last workgroup to leave advances the counter (skipping the value whose
// successor would be 0, so that a tag is never 0 and two launches in a row never
// share one), re-arms the chunk counter and flips the bank of share claims the
// next launch uses; each launch clears the other bank while it runs.
#include "attend_dev.h"
#include "sketch_dev.h"

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
    unsigned long long *claims;  // [2][kMaxStepGrid * kClaimStride]: a share is taken when
                                 // its word's low 32 bits go from 0 to 1
    // with sketches (NULL hdr otherwise): the sketch rows and the exact-score
    // area of a unit that scores every block (the unit kernel); per unit the
    // number of blocks whose fp32 row the selection read, or NULL
    skt::SketchArgs k;
    int32_t *cand_counts;
    uint32_t spin_limit;         // bound of a phase-2 wait (polls)
    uint32_t test_flags;         // bit 0: owners leave their shares unclaimed; bits 1, 2:
                                 // the unit kernel always / never (tests only)
    int B, units, nsplit;
};

constexpr int kStageBlocks = 1;  // attention pipeline stage: one block
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
#ifndef BTK_STEP_SEGMENT_COST
#define BTK_STEP_SEGMENT_COST 520
#endif
constexpr int kSegmentCost = BTK_STEP_SEGMENT_COST;
// With sketches (the unit kernel): candidates (blocks whose sketch interval
// reaches the threshold) scored exactly from LDS; beyond, every block is scored.
constexpr int kStepCand = 1024;
constexpr int kRowPer = kRun / kThreads;  // block-table entries per thread (phase 2)
// The unit kernel's block limit per sequence: its intervals, page ids and
// touched-block scores sit in LDS (16 bytes a block, 48 KB at 3072 blocks),
// leaving two workgroups per CU at D = 128 bf16.  Tables a little wider than
// a power of two (a slot kept for the next page) stay within it.
constexpr int kUnitRun = 3072;
constexpr int kUnitRowPer = kUnitRun / kThreads;
constexpr int step_qn(int D) { return (kMaxGroup * D + kThreads - 1) / kThreads; }
// The last 1/kStealFrac of the rows is handed out in chunks of kStealRows to the
// workgroups that finish their static share first.
#ifndef BTK_STEP_STEAL_FRAC
#define BTK_STEP_STEAL_FRAC 8
#endif
#ifndef BTK_STEP_STEAL_ROWS
#define BTK_STEP_STEAL_ROWS 256
#endif
constexpr int kStealFrac = BTK_STEP_STEAL_FRAC;
// Sequences whose row prefix a workgroup holds in LDS at once; a larger batch is
// walked window by window (the prologue keeps only each window's first row).
constexpr int kWin = 1024;
static_assert(kWin % kThreads == 0 && kMaxStepBatch % kWin == 0, "window shape");
constexpr uint32_t kStealRows = BTK_STEP_STEAL_ROWS;

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

// A sequence length as the step uses it: -1 when out of range (its unit then
// writes -1 indices and flags the error).
__device__ __forceinline__ int valid_len(int L, int max_blocks) {
    return L >= 1 && L <= max_blocks * kPage ? L : -1;
}
// Rows of a sequence's units in the share cut: per unit kSegmentCost charged
// rows, then one per block (one placeholder row for an invalid length).
__device__ __forceinline__ uint32_t unit_rows(int L, int Hkv) {
    return (uint32_t)Hkv * ((uint32_t)kSegmentCost + (uint32_t)(L >= 0 ? (L + kPage - 1) / kPage : 1));
}
// The position whose block the step refreshes (S1): with the KV append the
// newest token, else first_pos (none when it is NULL or the length is invalid).
template <bool APPEND>
__device__ __forceinline__ int touched_pos(const StepArgs &a, int b, int L) {
    if (APPEND) return L >= 0 ? L - 1 : -1;
    return a.s.first_pos ? a.s.first_pos[b] : -1;
}

// Loads the row prefix of sequences [base, base + wlen) into LDS, rows before
// the window being `first` (workgroup-uniform call).
template <bool APPEND>
__device__ __forceinline__ void load_window(const StepArgs &a, int base, int wlen, uint32_t first,
                            uint32_t *rows, int *lens, int *fps, int *scan_red) {
    constexpr int kPer = kWin / kThreads;
    const int tid = threadIdx.x;
    __syncthreads();  // the previous window is no longer read
    int Ls[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)  // all in flight together
        Ls[i] = i * kThreads + tid < wlen ? a.s.seq_lens[base + i * kThreads + tid] : 0;
    uint32_t carry = first;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int w = i * kThreads + tid;
        uint32_t n = 0;
        if (w < wlen) {
            const int L = valid_len(Ls[i], a.s.max_blocks);
            n = unit_rows(L, a.s.Hkv);
            lens[w] = L;
            fps[w] = touched_pos<APPEND>(a, base + w, L);
        }
        const uint32_t before = carry + (uint32_t)sel::wg_exclusive_scan((int)n, scan_red);
        if (w < wlen) {
            rows[w] = before;
            if (w == wlen - 1) rows[w + 1] = before + n;
        }
        carry += (uint32_t)(scan_red[0] + scan_red[1] + scan_red[2] + scan_red[3]);
    }
    __syncthreads();
}

// APPEND: the KV append of the step is fused in (a separate instantiation, so
// that the plain step carries none of its code).  SPLITS: the attention of a
// unit may be split over several items (instances without it carry no split
// merge, whose code alone made the one-split step slower).

template <typename T, int D, bool APPEND, bool SPLITS>
__global__ __launch_bounds__(kThreads, 2) void decode_step_kernel(StepArgs a) {
    __shared__ float qs[D];
    __shared__ int pages[kRun];
    __shared__ float sc_lds[kRun];
    __shared__ int flag;
    // read as 16-byte vectors (histogram bins, candidate keys): 16-byte aligned
    __shared__ __align__(16) uint32_t hist[sel::kTopkPasses * sel::kHistWords];
    __shared__ __align__(16) uint32_t cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ __align__(16) float crow[kWaves * D];
    __shared__ __align__(16) uint32_t newtok[APPEND ? D * sizeof(T) / 4 : 4];  // new key
    // the row prefix of one window of kWin sequences, [base, base + wlen)
    __shared__ uint32_t rows[kWin + 1];  // centroid rows before each sequence, then the window end
    __shared__ int lens[kWin];           // sequence lengths, -1: invalid
    __shared__ int fps[kWin];            // decode positions (first touched token)
    __shared__ uint32_t wrows[kMaxStepBatch / kWin + 1];  // rows before each window, then R
    __shared__ int item_s, owns_s;
    __shared__ uint32_t tag_s, bank_s;
    // queries while scoring, top-k keys of long contexts, attention merges
    extern __shared__ float dyn[];
    sel::ScoreSmem sm{dyn, qs, pages, sc_lds, &flag, newtok};
    sel::TopkSmem tk{hist, cand, red, scan_red, reinterpret_cast<uint32_t *>(dyn)};
    const int tid = threadIdx.x;
    const int Hkv = a.s.Hkv;

    // Thread 0 fetches the launch tag and the claim bank and, in the same round
    // trip, claims this workgroup's share in both banks (the bank is not known
    // yet); its word in the bank this launch does not use is cleared again
    // afterwards, so that the next launch finds it at zero.  Meanwhile the row
    // prefix is built: per unit kSegmentCost charged rows, then one row per
    // block (a single placeholder row for an invalid length, which writes -1
    // indices and flags the error).
    unsigned long long *const mine = a.claims + (size_t)blockIdx.x * kClaimStride;
    unsigned long long own0 = 1ull, own1 = 1ull;
    uint32_t tag0 = 0u, bank0 = 0u;
    if (tid == 0) {
        tag0 = __hip_atomic_load(&a.queue[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bank0 = __hip_atomic_load(&a.queue[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!(a.test_flags & 1u)) {
            own0 = __hip_atomic_fetch_add(mine, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            own1 = __hip_atomic_fetch_add(mine + (size_t)kMaxStepGrid * kClaimStride, 1ull,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // (Sequences past the first window only add to the window totals; a window
    // is loaded when a share first reaches its rows.)
    {
        int Lc = tid < a.B ? a.s.seq_lens[tid] : 0;
        uint32_t carry = 0u;  // rows before b0
        for (int b0 = 0; b0 < a.B; b0 += kThreads) {
            const int b = b0 + tid;
            // the next lengths are in flight during this scan
            const int Ln = b + kThreads < a.B ? a.s.seq_lens[b + kThreads] : 0;
            uint32_t n = 0;
            if (b < a.B) {
                const int L = valid_len(Lc, a.s.max_blocks);
                n = unit_rows(L, Hkv);
                if (b < kWin) {
                    lens[b] = L;
                    fps[b] = touched_pos<APPEND>(a, b, L);
                }
            }
            const uint32_t before = carry + (uint32_t)sel::wg_exclusive_scan((int)n, scan_red);
            if (b < a.B && b < kWin) {
                rows[b] = before;
                if (b == min(a.B, kWin) - 1) rows[b + 1] = before + n;
            }
            if (b < a.B && b % kWin == 0) wrows[b / kWin] = before;
            if (b == a.B - 1) wrows[(a.B + kWin - 1) / kWin] = before + n;
            carry += (uint32_t)(scan_red[0] + scan_red[1] + scan_red[2] + scan_red[3]);
            Lc = Ln;
        }
    }
    if (tid == 0) {
        const uint32_t bank = bank0 & 1u;
        tag_s = tag0 + 1u;
        bank_s = bank;
        owns_s = (bank ? own1 : own0) == 0ull;
        // this workgroup's word of the other bank (no other workgroup touches it)
        __hip_atomic_store(mine + (size_t)(bank ^ 1u) * kMaxStepGrid * kClaimStride, 0ull,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t tag = tag_s, bank = bank_s;
    unsigned long long *claims = a.claims + (size_t)bank * kMaxStepGrid * kClaimStride;
    {  // the other bank's words that no workgroup of this grid owns
        unsigned long long *other = a.claims + (size_t)(bank ^ 1u) * kMaxStepGrid * kClaimStride;
        for (uint32_t w = gridDim.x + blockIdx.x * kThreads + tid; w < (uint32_t)kMaxStepGrid;
             w += gridDim.x * kThreads)
            __hip_atomic_store(other + (size_t)w * kClaimStride, 0ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    const int total = a.units * a.nsplit;  // phase-2 items

    // ---- phase 1: this workgroup's static share of the first rows (if it
    // claimed it), then chunks of the rest while any are left (shares end at
    // different times: the workgroups that finish first take more of the rest),
    // then, in a workgroup that holds no phase-2 item, any share still unclaimed
    const int nwin = (a.B + kWin - 1) / kWin;
    const uint64_t R = wrows[nwin];
    const uint64_t RS = R - R / kStealFrac;
    int base = 0, wlen = min(a.B, kWin);  // the window in LDS
    uint32_t r = 0, r1 = 0;
    if (owns_s) {
        r = (uint32_t)(RS * blockIdx.x / gridDim.x);
        r1 = (uint32_t)(RS * (blockIdx.x + 1) / gridDim.x);
    }
    bool chunks_left = true;
    int b = 0;
    for (;;) {
        if (r >= r1 && chunks_left) {
            if (tid == 0) item_s = (int)atomicAdd(a.steal, 1u);
            __syncthreads();
            const uint64_t c0 = RS + (uint64_t)item_s * kStealRows;
            __syncthreads();  // item_s is written again
            if (c0 < R) {
                r = (uint32_t)c0;
                r1 = (uint32_t)min(R, c0 + kStealRows);
            } else {
                chunks_left = false;
            }
        }
        if (r >= r1) {
            if ((int)blockIdx.x < total && blockIdx.x != 0) break;
            // workgroup 0, or one without items: take a share whose workgroup has
            // not started (the
            // lowest unclaimed one; thread 0 claims it, another look if that fails)
            if (tid == 0) item_s = 0x7fffffff;
            __syncthreads();
            for (uint32_t v = tid; v < gridDim.x; v += kThreads)
                if (__hip_atomic_load(claims + (size_t)v * kClaimStride, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == 0ull)
                    atomicMin(&item_s, (int)v);
            __syncthreads();
            if (tid == 0 && item_s != 0x7fffffff &&
                __hip_atomic_fetch_add(claims + (size_t)item_s * kClaimStride, 1ull,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0ull)
                item_s = -2;  // taken meanwhile: look again
            __syncthreads();
            const int v = item_s;
            __syncthreads();  // item_s is written again
            if (v == -2) continue;
            if (v == 0x7fffffff) break;
            r = (uint32_t)(RS * (uint32_t)v / gridDim.x);
            r1 = (uint32_t)(RS * ((uint32_t)v + 1) / gridDim.x);
            b = 0;
            continue;
        }
        if (r < rows[0] || r >= rows[wlen]) {  // the rows of another window
            int k = 0;
            while (k + 1 < nwin && wrows[k + 1] <= r) ++k;
            base = k * kWin;
            wlen = min(a.B - base, kWin);
            load_window<APPEND>(a, base, wlen, wrows[k], rows, lens, fps, scan_red);
            b = 0;
        }
        if (rows[b] > r) b = 0;
        while (rows[b + 1] <= r) ++b;
        const int nb = lens[b] < 0 ? -1 : (lens[b] + kPage - 1) / kPage;
        constexpr uint32_t kCost = kSegmentCost;
        const uint32_t per_unit = kCost + (nb < 0 ? 1u : (uint32_t)nb);
        const uint32_t off = r - rows[b];
        const uint32_t g = off / per_unit, o = off % per_unit;  // o < kCost: charged rows
        const uint32_t e = min(per_unit, o + (r1 - r));         // this share's end in the unit
        const int j0 = (int)(o > kCost ? o - kCost : 0u);
        const int j1 = (int)(e > kCost ? e - kCost : 0u);
        if (j1 > j0) {
            sel::score_segment<T, D, kScanRows, kRun, APPEND>(
                a.s, base + b, (int)g, j0, j1, nb, lens[b], fps[b], sm, crow,
                a.ready + ((size_t)(base + b) * Hkv + g) * kReadyStride, tag);
            __syncthreads();  // LDS is reused by the next segment
        }
        r += e - o;
    }

    // ---- phase 2: (unit, split) items
    int32_t *list = reinterpret_cast<int32_t *>(sc_lds);  // the split's share, <= 256 entries
    // item i goes to workgroup i mod G: with fewer items than resident
    // workgroups the first G/2 take one each, one per CU (workgroups are
    // placed on CUs in index order), so no CU runs two attentions at once
    for (int item = (int)blockIdx.x;; item += (int)gridDim.x) {
        __syncthreads();  // LDS is reused
        if (item >= total) break;
        const int unit = item / a.nsplit, split = item % a.nsplit;
        const int bu = unit / Hkv;
        // the length from LDS when the sequence lies in the window held there
        const int L = bu >= base && bu < base + wlen ? lens[bu - base]
                                                     : valid_len(a.s.seq_lens[bu], a.s.max_blocks);
        const int nb = L < 0 ? -1 : (L + kPage - 1) / kPage;
        // the sequence's block-table row is requested before the wait, so that
        // the attention finds the selected blocks' pages in LDS
        const bool row_lds = nb >= 0 && nb <= kRun;
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
                if (++spins > a.spin_limit) {  // never expected: report, do not hang
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
        // through btk_decode_step_sketch: every block's fp32 row was read
        if (a.cand_counts && split == 0 && tid == 0)
            a.cand_counts[unit] = nb > a.s.top_k ? nb : 0;
        if (row_lds) {
#pragma unroll
            for (int i = 0; i < kRowPer; ++i)
                if (i * kThreads + tid < nb) pages[i * kThreads + tid] = prow[i];
        }
        // the appended token's cache stores are done before the block can be read
        if (APPEND) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        att::attend_item<T, D, att::kSelected, kStageBlocks, SPLITS>(
            a.t, unit, split, dyn, &flag, list, L < 0 ? 0 : L, row_lds ? pages : nullptr);
        __syncthreads();  // LDS is reused by the next item
    }
    // the last workgroup to leave re-arms the queue, flips the claim bank and
    // advances the counter
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&a.queue[1], 1u);
        if (prev == gridDim.x - 1) {
            __hip_atomic_store(&a.queue[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.steal, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.queue[3], bank ^ 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.queue[2], tag == 0xffffffffu ? 0u : tag, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// With sketches, when the units fill the device: one workgroup per (sequence,
// KV head) unit does the whole step for it, so no workgroup waits for another.
// The queries, the length, the block-table row (clamped to the table) and the
// first 256 sketch rows (likewise) are requested together, before the length
// is known; the unit's sketch rows are scanned into intervals held in LDS (the
// mean query is formed, and the touched block's keys are requested, while the
// first rows are in flight); then the touched blocks are refreshed (S1: centroid, exact score
// kept in LDS, sketch row), the threshold and the candidates taken from the
// intervals in LDS, the candidates scored exactly from their fp32 rows, the k
// best kept, and the unit attended.  Launch bounds 256 x 1: the kernel may use
// more registers than the persistent one (two workgroups per CU still fit at
// D = 128 bf16).  Limits (checked on the host): a block table of at
// most kUnitRun blocks, one attention split, top_k <= 256 and a
// group of at most 8 heads.  Results are those of the persistent form (the
// same arithmetic per unit, blocks in the same order).
// Sketch-row header loads per lane per scan stage: 1, two stages of 256 rows in
// flight per workgroup.  With every CU scanning at once the memory system is
// saturated, and more requests in flight only lengthen each one: 2 (512-row
// stages) took the Qwen3-8B-shaped step from 37.8 to 41.1 us.  Likewise the
// attention keeps the two one-block stages per wave of the persistent kernel
// (four or six stages: 11.8 / 13.0 instead of 10.0 us per unit).
#ifndef BTK_UNIT_HK
#define BTK_UNIT_HK 1
#endif
// Radix passes of the threshold: any lower bound of the k-th largest lower end
// keeps every block that can be selected, so the search may stop at the
// threshold bin's lower edge.  After two passes the candidates are those of the
// exact threshold (50 mean, 69 at most on the Qwen3-8B-shaped layer); after one
// they were 63 / 242 and the longer rescore and rank cost more than the pass.
#ifndef BTK_UNIT_TPASSES
#define BTK_UNIT_TPASSES 2
#endif

// The unit kernel's S1: waves 1-3 refresh the touched blocks jt + w - 1,
// jt + w + 2, ... below j1 (centroid from the keys, stored; exact score as the
// full scan computes it, into kex[j - jt] in LDS; sketch row rebuilt).  kt
// holds the keys of the wave's first touched block (page pw), requested before
// the scan.
template <typename T, int D>
__device__ __forceinline__ void unit_refresh(const StepArgs &a, int unit, int b, int L, int j1,
                                             int jt, int pw, KeyTile<T, D> &kt,
                                             const float *qs, float *crow, float *kex) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int g = unit % a.s.Hkv;
    const int32_t *bt_row = a.s.bt + (size_t)b * a.s.max_blocks;
    const T *keys = static_cast<const T *>(a.s.k_cache) + (size_t)g * kPage * D;
    const size_t page_stride = (size_t)a.s.Hkv * kPage * D;
    constexpr int kRefWaves = kWaves - 1, E = D / kWave, VPL = D / 16;
    const int jw = wave == 0 ? j1 : jt + wave - 1;
    float qf[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) qf[e] = qs[(lane % 16) * VPL + e];
    const size_t urow = (size_t)unit * a.s.max_blocks;
    for (int j = jw; j < j1; j += kRefWaves) {
        const int page = j == jw ? pw : bt_row[j];
        if (page < 0 || page >= a.s.num_pages) {  // scored (and flagged) as -inf
            if (lane == 0) kex[j - jt] = -INFINITY;
            continue;
        }
        const int v = min(kPage, L - j * kPage);
        float *row_lds = crow + wave * D;
        if (j != jw) kt.load(keys + (size_t)page * page_stride, v, lane);
        kt.mean_to(v, a.s.cent_out + ((size_t)page * a.s.Hkv + g) * D, row_lds, true, lane);
        __builtin_amdgcn_wave_barrier();
        floatx4_t cv[VPL / 4];
#pragma unroll
        for (int vv = 0; vv < VPL / 4; ++vv)
            cv[vv] = reinterpret_cast<const floatx4_t *>(row_lds + (lane % 16) * VPL)[vv];
        const float sc = sel::row16_sum(sel::row_partial<VPL>(qf, cv));
        if (lane == 0) kex[j - jt] = sc;
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = row_lds[lane * E + e];
        skt::encode_row<D>(x, page, urow + j, a.k.hdr, a.k.codes, lane);
        __builtin_amdgcn_wave_barrier();
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void decode_step_unit_kernel(StepArgs a) {
    __shared__ float qs[D];
    __shared__ int pages[kUnitRun];
    __shared__ float lo_lds[kUnitRun], hi_lds[kUnitRun];  // interval ends; then candidates
    __shared__ float kex[kUnitRun];                        // exact scores of the touched blocks
    __shared__ int flag;
    // read as 16-byte vectors (histogram bins, candidate keys): 16-byte aligned
    __shared__ __align__(16) uint32_t hist[sel::kTopkPasses * sel::kHistWords];
    __shared__ __align__(16) uint32_t cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ __align__(16) float crow[kWaves * D];
    __shared__ int32_t list[4 * kWave];  // the selection (top_k <= 256)
    __shared__ float qsum[2];
    __shared__ int ctot;
    extern __shared__ float dyn[];  // queries, then the attention's wave merge
    sel::ScoreSmem sm{dyn, qs, pages, lo_lds, &flag, nullptr};
    sel::TopkSmem tk{hist, cand, red, scan_red, reinterpret_cast<uint32_t *>(dyn)};
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, Hkv = a.s.Hkv;
    const int unit = (int)blockIdx.x, b = unit / Hkv, g = unit % Hkv;
    const int r = a.s.Hq / Hkv;
    // the queries, the length and the decode position, requested together
    const T *qp = static_cast<const T *>(a.s.q) + ((size_t)b * a.s.Hq + (size_t)g * r) * D;
    float qv[step_qn(D)];
#pragma unroll
    for (int k = 0; k < step_qn(D); ++k)
        qv[k] = sel::load_q<T>(qp + min(k * kThreads + tid, r * D - 1));
    const int Lraw = a.s.seq_lens[b];
    const int fpraw = a.s.first_pos ? a.s.first_pos[b] : -1;
    const int32_t *bt_row = a.s.bt + (size_t)b * a.s.max_blocks;
    // the block-table row, clamped to the table (requested before the length is known)
    int32_t prow[kUnitRowPer];
#pragma unroll
    for (int i = 0; i < kUnitRowPer; ++i)
        prow[i] = i < kRowPer || i * kThreads < a.s.max_blocks
                      ? bt_row[min(i * kThreads + tid, a.s.max_blocks - 1)] : 0;
    int L = -1, fp = -1, nb = 0, jt = 0, jw = 0, pw = -1;
    KeyTile<T, D> kt;
    skt::scan_sketch<D, BTK_UNIT_HK>(a.s, a.k, b, g, 0, a.s.max_blocks, [&] {
        L = valid_len(Lraw, a.s.max_blocks);
        fp = L >= 0 ? fpraw : -1;
        nb = L >= 0 ? (L + kPage - 1) / kPage : 0;
        jt = a.s.first_pos && fp >= 0 && fp < L ? fp / kPage : nb;
        return make_int2(nb, jt);
    }, sm.qs, qsum, lo_lds, hi_lds, [&] {
#pragma unroll
        for (int k = 0; k < step_qn(D); ++k)
            if (k * kThreads + tid < r * D) sm.qraw[k * kThreads + tid] = qv[k];
#pragma unroll
        for (int i = 0; i < kUnitRowPer; ++i)
            if (i * kThreads + tid < nb) pages[i * kThreads + tid] = prow[i];
        __syncthreads();
        // this wave's first touched block's page (from LDS) and keys
        jw = wave == 0 ? nb : jt + wave - 1;
        pw = jw < nb ? pages[jw] : -1;
        if (pw >= 0 && pw < a.s.num_pages)
            kt.load(static_cast<const T *>(a.s.k_cache) +
                        ((size_t)pw * Hkv + g) * kPage * D,
                    min(kPage, L - jw * kPage), lane);
        sel::mean_query<D>(a.s, sm);
        __syncthreads();
        skt::query_sums<D>(sm.qs, qsum);
        __syncthreads();
    });
    if (L < 0) {  // -1 indices, the error flagged; no output (as the persistent form)
        for (int i = tid; i < a.s.top_k; i += kThreads)
            a.s.indices[(size_t)unit * a.s.top_k + i] = -1;
        if (tid == 0) {
            flag_error(a.s.err, kErrSeqLen);
            if (a.cand_counts) a.cand_counts[unit] = 0;
        }
        return;
    }
    // S1 for the touched blocks, then S3
    unit_refresh<T, D>(a, unit, b, L, nb, jt, pw, kt, sm.qs, crow, kex);
    __syncthreads();
    int32_t *idx = a.s.indices + (size_t)unit * a.s.top_k;
    const int kb = min(a.s.top_k, nb);
    int32_t *cmap = reinterpret_cast<int32_t *>(lo_lds);  // (the ends are read first)
    float *cex = hi_lds;
    int m = 0;  // candidates, scored exactly
    __builtin_amdgcn_s_setprio(3);
    if (kb == nb) {  // every block is kept (no score is read)
        sel::select_topk(skt::LdsScores{hi_lds}, nb, a.s.top_k, sel::TopkOut{idx, list, 0, a.s.top_k},
                         tk);
    } else {
        m = skt::threshold_candidates<true, BTK_UNIT_TPASSES>(lo_lds, hi_lds, nb, kb, cmap,
                                                              kStepCand, tk, tk.cand, &ctot);
        if (m <= kStepCand) {
            skt::rescore<D, true>(a.s, b, g, cmap, m, pages, true, sm.qs, cex, kex, jt);
            __syncthreads();
        }
        sel::TopkOut o{idx, list, 0, a.s.top_k};
        o.map = cmap;
        o.mapped = true;
        if (m <= kThreads)
            skt::select_ranked(cex, m, a.s.top_k, o, tk.hist, tk.red);
        else if (m <= kStepCand)
            sel::select_topk(skt::LdsScores{cex}, m, a.s.top_k, o, tk);
        else {  // every block, with the full scan's code (the touched blocks again)
            sel::SelectArgs ax = a.s;
            ax.scores = a.k.exact;
            const size_t urow = (size_t)unit * a.s.max_blocks;
            __syncthreads();  // pages and lo_lds are free
            for (int i = tid; i < nb; i += kThreads) pages[i] = bt_row[i];
            __syncthreads();
            sel::check_pages(a.s, sm, nb);
            __syncthreads();
            sel::scan_rows<T, D, kScanRows, true>(ax, b, g, 0, nb, L, fp, sm, crow);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the scores are stored
            __syncthreads();
            sel::select_topk(sel::PlainScores{a.k.exact + urow}, nb, a.s.top_k,
                             sel::TopkOut{idx, list, 0, a.s.top_k}, tk);
            m = nb;
            __syncthreads();
            for (int i = tid; i < nb; i += kThreads) pages[i] = bt_row[i];  // for the attention
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (tid == 0 && a.cand_counts) a.cand_counts[unit] = m;
    __syncthreads();
    // S4
    att::attend_item<T, D, att::kSelected, kStageBlocks, false>(a.t, unit, 0, dyn, &flag, list,
                                                                L, pages);
}

// CUs of the current device (cached per device), or 0 on error.
int device_cus() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int &c = cached[dev & 63];
    if (c == 0 && hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        c = 0;
    return c;
}

template <typename T, int D>
hipError_t launch_unit(const Dims &d, const StepArgs &a, hipStream_t stream) {
    const size_t r = d.group();
    size_t n = r * D;                                                 // queries
    const size_t wave_merge = (size_t)att::kWaves * r * D + 2 * att::kWaves * 16;
    n = n > wave_merge ? n : wave_merge;
    if (d.max_blocks > 32 * kWave && n < 512) n = 512;  // top-k bitmaps beyond 2048 blocks
    hipLaunchKernelGGL((decode_step_unit_kernel<T, D>), dim3((unsigned)a.units), dim3(kThreads),
                       sizeof(float) * n, stream, a);
    return hipGetLastError();
}

// The unit kernel serves problems whose units fill the device (at least one per
// CU) and fit its limits; test_flags bit 1 / bit 2 force it on / off.
bool use_unit_kernel(const Dims &d, const AttendPlan &ap, int top_k, uint32_t test_flags) {
    const bool fits = d.max_blocks <= kUnitRun && ap.nsplit_max == 1 && top_k <= 4 * kWave &&
                      d.group() <= 8;
    if (!fits || (test_flags & 4u)) return false;
    if (test_flags & 2u) return true;
    const int cus = device_cus();
    return cus > 0 && (long)d.B * d.Hkv >= cus;
}

size_t step_lds_floats(const Dims &d, const AttendPlan &ap) {
    const size_t r = d.group();
    size_t n = r * d.D;                                              // queries
    const size_t wave_merge = (size_t)att::kWaves * r * d.D + 2 * att::kWaves * 16;
    const size_t split_merge = 2 * (size_t)ap.nsplit_max * r + r;
    n = n > wave_merge ? n : wave_merge;
    n = n > split_merge ? n : split_merge;
    if (d.max_blocks > 32 * kWave && n < 512) n = 512;  // top-k bitmaps beyond 2048 blocks
    return n;
}

// resident workgroups of the step kernel on this device (cached per device)
template <typename T, int D, bool APPEND, bool SPLITS>
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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, decode_step_kernel<T, D, APPEND, SPLITS>, kThreads, lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[slot][0] = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (cached[slot][0] > kMaxStepGrid) cached[slot][0] = kMaxStepGrid;
    cached[slot][1] = (int)lds;
    *out = cached[slot][0];
    return hipSuccess;
}

template <typename T, int D, bool APPEND, bool SPLITS>
hipError_t launch_instance(size_t lds, const StepArgs &a, hipStream_t stream) {
    int grid = 0;
    const hipError_t e = resident_workgroups<T, D, APPEND, SPLITS>(lds, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_step_kernel<T, D, APPEND, SPLITS>), dim3(grid), dim3(kThreads),
                       lds, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch(const Dims &d, const SelectPlan &sp, const AttendPlan &ap, StepArgs a,
                  hipStream_t stream) {
    const size_t lds = sizeof(float) * step_lds_floats(d, ap);
    const bool splits = ap.nsplit_max > 1;
    if (a.k.hdr && use_unit_kernel(d, ap, a.s.top_k, a.test_flags))
        return launch_unit<T, D>(d, a, stream);
    if (a.k.hdr) {  // too few units: the persistent fp32 scan, keeping the sketch current
        a.s.sk_hdr = a.k.hdr;
        a.s.sk_codes = a.k.codes;
    }
    if (a.s.k_new)
        return splits ? launch_instance<T, D, true, true>(lds, a, stream)
                      : launch_instance<T, D, true, false>(lds, a, stream);
    return splits ? launch_instance<T, D, false, true>(lds, a, stream)
                  : launch_instance<T, D, false, false>(lds, a, stream);
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
                              unsigned long long *claims, uint32_t spin_limit,
                              uint32_t test_flags, uint32_t *err, hipStream_t stream,
                              const void *k_new, const void *v_new, void *sketch,
                              float *sk_lo, float *sk_hi, int32_t *cand_counts) {
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
    a.k = skt::SketchArgs{nullptr, nullptr, nullptr, nullptr, nullptr};
    a.cand_counts = nullptr;
    if (sketch) {  // the score area holds exact scores of units scored whole
        skt::SketchHdr *hdr = static_cast<skt::SketchHdr *>(sketch);
        a.k = skt::SketchArgs{hdr, reinterpret_cast<uint8_t *>(hdr) + sketch_rows_offset(d),
                              sk_lo, sk_hi, scores};
        a.cand_counts = cand_counts;
    }
    a.ready = ready;
    a.queue = queue;
    a.steal = steal;
    a.claims = claims;
    a.spin_limit = spin_limit;
    a.test_flags = test_flags;
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
