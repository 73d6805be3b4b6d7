// Device code of the block sketches, shared by the stand-alone sketch kernels
// (sketch.hip) and the single-launch decode step with sketches (step.hip).
// (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What carries
// the argument": blocks are scored by their averaged keys and the k best are
// kept.  A sketch changes which centroid rows are read, not which blocks are
// selected.)
//
// A sketch row is an 8-bit copy of one block's fp32 centroid, kept per sequence
// in block-table order, so that a unit's sketch is one contiguous stream:
//   header[i] = {page + 1 (0: no sketch), scale = amax / 127}
//   codes[i][d] = rint(c_d / scale) + 128  (in 1 .. 255; 128 when amax = 0)
// for row i = (b * Hkv + g) * max_blocks + j (block j of sequence b, KV head g).
//
// Why a selection through the sketch keeps exactly the same blocks.  With c the
// fp32 centroid, qs the scaled mean query and s = qs . c, the sketch gives
// sa = scale * (sum_d qs_d * code_d - 128 * sum_d qs_d).  Rounding c_d / scale
// to an integer moves each term by at most 0.50001 * scale * |qs_d| (the fp32
// quotient is within 127 * 2^-24 of exact), and the fp32 evaluation of either
// sum, in any order, by at most 127 * 2^-24 * (255 + 128) * scale * |qs|_1
// (the sketch's) and 127 * 2^-24 * 127 * scale * |qs|_1 (the exact score's),
// about 0.004 * scale * |qs|_1 together.  So every score s computed by the
// fp32 scan lies in [sa - e, sa + e] with e = 0.51 * scale * |qs|_1 (the margin
// also covers the rounding of sa - e and sa + e themselves).  With tau the
// kb-th largest lower end, at least kb blocks score at least tau; a block whose
// upper end is below tau therefore scores below kb others and cannot be
// selected under any tie rule.  The remaining candidates are scored exactly as
// the full scan scores them (the same arithmetic, the same bits) and the top kb
// of those are selected with the same tie rule, so the indices equal those of
// the full scan.  A row whose header does not name the block's current page
// (not built, stale, invalid page) and a block refreshed in the same call are
// always candidates.
#pragma once
#include "select_dev.h"

namespace btk {
namespace skt {

using sel::kThreads;
using sel::kWaves;


constexpr float kBoundFactor = 0.51f;

struct SketchArgs {
    SketchHdr *hdr;   // [units * max_blocks] (written only by refreshes)
    uint8_t *codes;   // [units * max_blocks][D]
    float *lo, *hi;   // [units * max_blocks] interval ends (workspace)
    float *exact;     // [units * max_blocks] exact scores when every block is scored (workspace)
};


// Scores read from LDS (see sel::PlainScores).
struct LdsScores {
    const float *sc;  // [nb]
    template <int N>
    __device__ __forceinline__ void fill(uint32_t (&bits)[N], int first, int stride, int nb) const {
#pragma unroll
        for (int i = 0; i < N; ++i)
            bits[i] = i * stride + first < nb ? __float_as_uint(sc[i * stride + first]) : 0u;
    }
};

// The scaled mean query's sums for the bound: q128 = 128 * sum(qs), qn1 =
// sum |qs| (wave 0 computes them into out[0], out[1]; the caller synchronises).
template <int D>
__device__ __forceinline__ void query_sums(const float *qs, float *out) {
    const int tid = threadIdx.x;
    if (tid < kWave) {
        float s0 = 0.f, s1 = 0.f;
        for (int d = tid; d < D; d += kWave) {
            s0 += qs[d];
            s1 += fabsf(qs[d]);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            s0 += __shfl_xor(s0, off);
            s1 += __shfl_xor(s1, off);
        }
        if (tid == 0) {
            out[0] = 128.f * s0;
            out[1] = s1;
        }
    }
}

// The threshold and the candidates of one unit, over the workgroup: tau is
// the kb-th largest lower end (order-preserving keys, as sel::score_key), the
// candidates are the blocks j < nb whose upper end's key is >= tau, written in
// ascending order to map[0 .. m) when m <= cap.  Returns m (workgroup-uniform).
// Up to 2048 blocks (KMAX <= 8) the lower and upper ends are requested
// together; beyond, the upper ends once tau is known (fewer registers).  The
// lower ends go through the radix passes of the four-wave top-k
// (sel::select_topk_wg4).  count: LDS of KMAX * kWaves words (may alias
// sm.cand), total: one LDS word.  LDS: the ends are in this workgroup's LDS
// (plain loads) instead of the workspace (agent-scope loads); every end is read
// before map is written (two barriers later), so map may alias lo_src.
// MAXP: at most that many radix passes; tau is then a lower bound of the kb-th
// largest lower end (the lower edge of its bin), which admits more candidates
// but keeps every block that can be selected.
template <int KMAX, bool LDS = false, int MAXP = sel::kTopkPasses>
__device__ __forceinline__ int threshold_candidates_wg4(const float *lo_src, const float *hi_src, int nb, int kb,
                                        int32_t *map, int cap, sel::TopkSmem &sm,
                                        uint32_t *count, int *total) {
    auto ld = [](const float *p) { return LDS ? *p : load_relaxed(p); };
    uint32_t *red = sm.red;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    for (int i = tid; i < sel::kTopkPasses * sel::kHistWords / 4; i += kThreads)
        reinterpret_cast<u32x4_t *>(sm.hist)[i] = u32x4_t{0u, 0u, 0u, 0u};
    constexpr bool kHiEarly = KMAX <= 8;
    uint32_t key[KMAX], hk[kHiEarly ? KMAX : 1];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {  // unconditional (clamped): all in flight together
        key[i] = __float_as_uint(ld(lo_src + min(i * kThreads + tid, nb - 1)));
        if constexpr (kHiEarly)
            hk[i] = __float_as_uint(ld(hi_src + min(i * kThreads + tid, nb - 1)));
    }
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int j = i * kThreads + tid;
        key[i] = j < nb ? score_key(__uint_as_float(key[i])) : 0u;
        kmin = j < nb ? min(kmin, key[i]) : kmin;
        kmax = max(kmax, key[i]);
    }
    // a lower bound of the result: for kb <= 64, in each wave the smallest of
    // the largest keys of its first kb lanes (0 if one of them holds none)
    const uint32_t bound = kb <= kWave ? (lane < kb ? kmax : 0xffffffffu) : kmin;
    const uint32_t wave_lo = ~sel::wave_max_u32(~bound);
    kmax = sel::wave_max_u32(kmax);
    if (lane == 0) {
        red[wave] = wave_lo;
        red[kWaves + wave] = kmax;
    }
    __syncthreads();
    uint32_t lo = kb <= kWave ? max(max(red[0], red[1]), max(red[2], red[3]))
                              : min(min(red[0], red[1]), min(red[2], red[3]));
    uint32_t hi = max(max(red[kWaves], red[kWaves + 1]), max(red[kWaves + 2], red[kWaves + 3]));
    int need = kb;
#pragma unroll 1
    for (int p = 0; p < MAXP && lo < hi; ++p) {
        uint32_t *hist = sm.hist + p * sel::kHistWords;
        const uint32_t span = hi - lo;
        const int shift = max(0, 24 - __builtin_clz(span));
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
            const uint32_t off = key[i] - lo;
            atomicAdd(&hist[off <= span ? (off >> shift) : 256u + lane], 1u);
        }
        __syncthreads();
        uint32_t in_bin;
        const uint32_t b_sel = sel::locate_bin(hist, need, lane, &in_bin);
        const uint32_t top = (b_sel << shift) + ((1u << shift) - 1u);
        if (top < span) hi = lo + top;
        lo += b_sel << shift;
        if (in_bin == (uint32_t)need && lo < hi) break;  // the bin is kept whole: tau = lo
    }
    // a bin kept whole: exactly kb keys are >= lo; else lo = hi = the kb-th key
    // (or, after MAXP passes, lo <= the kb-th key)
    const uint32_t tau = lo;

    // the candidates, in block order: a count per (slot, wave), an exclusive
    // prefix over them, then each flagged lane writes its place
    uint32_t flags = 0u;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const uint32_t hv = kHiEarly ? hk[kHiEarly ? i : 0]
                                     : __float_as_uint(ld(hi_src + min(i * kThreads + tid, nb - 1)));
        const bool f = i * kThreads + tid < nb && score_key(__uint_as_float(hv)) >= tau;
        flags |= (uint32_t)f << i;
        const uint64_t bal = __ballot(f);
        if (lane == 0) count[i * kWaves + wave] = (uint32_t)__popcll(bal);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix over (slot, wave) in block order
        constexpr int N = KMAX * kWaves;  // <= 128
        const uint32_t c0 = 2 * lane < N ? count[2 * lane] : 0u;
        const uint32_t c1 = 2 * lane + 1 < N ? count[2 * lane + 1] : 0u;
        const uint32_t incl = sel::wave_inclusive_scan(c0 + c1);
        const uint32_t excl = incl - (c0 + c1);
        if (2 * lane < N) count[2 * lane] = excl;
        if (2 * lane + 1 < N) count[2 * lane + 1] = excl + c0;
        if (lane == kWave - 1) *total = (int)incl;
    }
    __syncthreads();
    const int m = *total;
    if (m <= cap) {
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
            const bool f = (flags >> i) & 1u;
            const uint64_t bal = __ballot(f);
            if (f) {
                const int pos = (int)count[i * kWaves + wave] +
                                (int)__builtin_amdgcn_mbcnt_hi(
                                    (uint32_t)(bal >> 32),
                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                map[pos] = i * kThreads + tid;
            }
        }
    }
    __syncthreads();  // map, count, the histograms and red are read or reused next
    return m;
}

// Dispatch on nb (at most 32 keys per thread: 8192 blocks; ends in LDS: at
// most 4096 blocks), kb < nb.
template <bool LDS = false, int MAXP = sel::kTopkPasses>
__device__ __forceinline__ int threshold_candidates(const float *lo, const float *hi, int nb,
                                                    int kb, int32_t *map, int cap,
                                                    sel::TopkSmem &sm, uint32_t *count,
                                                    int *total) {
    if (nb <= 4 * kThreads)
        return threshold_candidates_wg4<4, LDS, MAXP>(lo, hi, nb, kb, map, cap, sm, count, total);
    if (nb <= 8 * kThreads)
        return threshold_candidates_wg4<8, LDS, MAXP>(lo, hi, nb, kb, map, cap, sm, count, total);
    if (LDS || nb <= 16 * kThreads)  // (the ends in LDS: at most 4096 blocks)
        return threshold_candidates_wg4<16, LDS, MAXP>(lo, hi, nb, kb, map, cap, sm, count, total);
    return threshold_candidates_wg4<32>(lo, hi, nb, kb, map, cap, sm, count, total);
}

// Interval ends of the sketch scores of blocks [j0, j0 + n) of unit (b, g)
// into lo_lds[0 .. n) and hi_lds[0 .. n) (LDS; see store_intervals).  LPR =
// D / 16 lanes hold a row (16 codes each), so a wave instruction covers RPW =
// 64 / LPR rows; a pipeline stage is KU = HK * LPR such instructions per lane,
// two stages in flight.  A row's header and page id are needed once per row,
// not once per lane: each lane loads those of HK rows of the stage (lane l:
// rows l and l + 64 in the wave's row order) and the lanes holding a row take
// its scale from there (a lane permute), so a stage costs 4 KU + 3 HK
// registers instead of 7 KU.  qs: the scaled mean query (LDS); qsum (LDS):
// q128 = 128 * sum(qs), qn1 = sum |qs|; both are read after prep(), which the
// scan calls (workgroup-uniformly) once its first stage is requested, so that
// the caller can form them while those rows are in flight.  The first stage's
// rows are clamped to cap rows (cap >= n, within the unit's rows) and only then
// is lens() called for (n, jforce), so a caller whose length is still in flight
// passes cap = the table width and reads the length in lens(); prep() runs only
// when n > 0.  Blocks j >= jforce (refreshed in this call) and rows whose header
// does not name the block's page get (-inf, +inf): always candidates.  Nothing is stored to memory inside the
// loop: stores count in the same in-order memory counter as the loads, so a
// store issued there would hold up the wait for the next stage's rows until it
// completed.
template <int D, int HK, typename Lens, typename Prep>
__device__ __forceinline__ void scan_sketch(const sel::SelectArgs &a, const SketchArgs &s, int b,
                                            int g, int j0, int cap, Lens &&lens, const float *qs,
                                            const float *qsum, float *lo_lds, float *hi_lds,
                                            Prep &&prep) {
    int n = cap, jforce = 0;  // (n: the first stage's clamp until lens() is read)
    constexpr int LPR = D / 16;          // lanes per row
    constexpr int RPW = kWave / LPR;     // rows per wave per load
    constexpr int KU = HK * LPR;         // load steps per stage: HK * 64 rows per wave
    constexpr int ROWS = kWaves * RPW * KU;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int part = lane % LPR, rsub = lane / LPR;
    const size_t urow = ((size_t)b * a.Hkv + g) * a.max_blocks;
    const int32_t *bt = a.bt + (size_t)b * a.max_blocks;
    float qf[16];
    float q128 = 0.f, ebase = 0.f;
    // row of load step u, row group rs, in a stage starting at base
    auto row_of = [&](int base, int u, int rs) { return base + u * kWaves * RPW + wave * RPW + rs; };
    struct Stage {
        u32x4_t c[KU];
        uint32_t h0[HK], h1[HK];
        int32_t pg[HK];
    };
    auto issue = [&](Stage &st, int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = min(row_of(base, u, rsub), n - 1);
            st.c[u] = *reinterpret_cast<const u32x4_t *>(s.codes + (urow + j0 + row) * D +
                                                         16 * part);
        }
#pragma unroll
        for (int h = 0; h < HK; ++h) {  // this lane's rows: step u = lane / RPW + h * LPR
            const int row = min(row_of(base, lane / RPW + h * LPR, lane % RPW), n - 1);
            const uint32_t *hp = reinterpret_cast<const uint32_t *>(s.hdr + urow + j0 + row);
            st.h0[h] = hp[0];
            st.h1[h] = hp[1];
            st.pg[h] = bt[j0 + row];
        }
    };
    auto reduce = [&](const Stage &st, int base) {
        // the scale of each of this lane's rows, or -1: always a candidate
        float sv[HK];
#pragma unroll
        for (int h = 0; h < HK; ++h) {
            const int row = row_of(base, lane / RPW + h * LPR, lane % RPW);
            const int page = st.pg[h];
            const bool valid = page >= 0 && page < a.num_pages && (int)st.h0[h] == page + 1 &&
                               j0 + row < jforce;
            const float sc = __uint_as_float(st.h1[h]);
            sv[h] = valid && sc < INFINITY ? sc : -1.f;  // (NaN and inf: candidates)
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = row_of(base, u, rsub);
            // this lane's 16 codes against its 16 query values, in a fixed order
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t cw = st.c[u][w];
                t = __builtin_fmaf(qf[4 * w + 0], (float)(cw & 0xffu), t);
                t = __builtin_fmaf(qf[4 * w + 1], (float)((cw >> 8) & 0xffu), t);
                t = __builtin_fmaf(qf[4 * w + 2], (float)((cw >> 16) & 0xffu), t);
                t = __builtin_fmaf(qf[4 * w + 3], (float)(cw >> 24), t);
            }
            // sum over the row's LPR lanes (quad xor 1, quad xor 2, half-row mirror)
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                               0, __builtin_bit_cast(int, t), 0xB1, 0xF, 0xF, false));
            t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                               0, __builtin_bit_cast(int, t), 0x4E, 0xF, 0xF, false));
            if constexpr (LPR == 8)
                t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                   0, __builtin_bit_cast(int, t), 0x141, 0xF, 0xF,
                                                   false));
            // the lane that loaded this row's header: (u % LPR) * RPW + rsub, slot u / LPR
            const float scale = __shfl(sv[u / LPR], (u % LPR) * RPW + rsub);
            const float sa = scale * (t - q128);
            const float e = scale * ebase;
            if (part == 0 && row < n) {
                lo_lds[row] = scale >= 0.f ? sa - e : -INFINITY;
                hi_lds[row] = scale >= 0.f ? sa + e : INFINITY;
            }
        }
    };
    Stage sa_, sb_;
    if (cap > 0) issue(sa_, 0);
    {
        const int2 nj = lens();
        n = nj.x;
        jforce = nj.y;
    }
    if (n > 0) {
        prep();
#pragma unroll
        for (int e = 0; e < 16; ++e) qf[e] = qs[16 * part + e];
        q128 = qsum[0];
        ebase = kBoundFactor * qsum[1];
        for (int base = 0;;) {
            issue(sb_, base + ROWS);
            reduce(sa_, base);
            base += ROWS;
            if (base >= n) break;
            issue(sa_, base + ROWS);
            reduce(sb_, base);
            base += ROWS;
            if (base >= n) break;
        }
    }
}

// The k best of m <= 256 candidate scores sc[0 .. m) (LDS, in ascending block
// order), by rank, over the workgroup: candidate t is kept when fewer than
// kb = min(top_k, m) candidates beat it, a candidate beating t when its score
// is larger or equal with a lower index (equal scores go to the lower block;
// -0.0 equals +0.0).  This is the rule of sel::select_topk, so the same blocks
// are kept; they are written in ascending order through out (which maps
// candidate numbers to blocks), then -1 up to top_k.  Each candidate's rank
// key is 64 bits, its score key above the complement of its number, so that
// "beats" is one unsigned comparison.  keys: 512 LDS words, 16-byte aligned
// (may alias sm.hist), wcount: kWaves LDS words (may alias sm.red).
__device__ __forceinline__ void select_ranked(const float *sc, int m, int top_k,
                                              const sel::TopkOut &out, uint32_t *keys,
                                              uint32_t *wcount) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int kb = min(top_k, m);
    const uint64_t mine =
        tid < m ? ((uint64_t)score_key(sc[tid]) << 32) | (uint64_t)(~(uint32_t)tid) : 0ull;
    reinterpret_cast<uint64_t *>(keys)[tid] = mine;  // candidates from m on hold 0
    __syncthreads();
    int beat = 0;
    // 32 keys (sixteen LDS reads in flight) at a time; keys past m hold 0 and
    // beat no candidate
    for (int c = 0; c < (m + 31) / 32; ++c) {
        u32x4_t k4[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) k4[q] = reinterpret_cast<const u32x4_t *>(keys)[16 * c + q];
#pragma unroll
        for (int q = 0; q < 16; ++q)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint64_t k = ((uint64_t)k4[q][2 * e + 1] << 32) | k4[q][2 * e];
                beat += k > mine ? 1 : 0;
            }
    }
    const bool keep = tid < m && beat < kb;
    const uint64_t bal = __ballot(keep);
    if (lane == 0) wcount[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    for (int w = 0; w < wave; ++w) pos += (int)wcount[w];
    if (keep) out.put(pos, tid);
    for (int i = kb + tid; i < top_k; i += kThreads) out.put(i, -1);
    __syncthreads();  // keys and wcount are reused
}

// Stores the n interval ends staged by scan_sketch for blocks [j0, j0 + n) of
// the unit whose rows start at urow, contiguously, with agent-scope stores (the
// unit's selection may run in a workgroup on another XCD).  Called with the
// staged values visible to every thread; ends with the stores issued.
__device__ __forceinline__ void store_intervals(const SketchArgs &s, size_t urow, int j0, int n,
                                                const float *lo_lds, const float *hi_lds) {
    for (int i = threadIdx.x; i < n; i += kThreads) {
        store_relaxed(s.lo + urow + j0 + i, lo_lds[i]);
        store_relaxed(s.hi + urow + j0 + i, hi_lds[i]);
    }
}

// Exact scores of the m blocks map[0 .. m) of unit (b, g) into sc[0 .. m)
// (LDS), with the full scan's arithmetic (sel::row_partial, sel::row16_sum;
// 16 lanes per centroid row), so each equals the full scan's score bit for bit;
// an out-of-range page scores -inf and sets the error bit, as in the full scan.
// Page ids come from pages[map[i]] (LDS, the block-table row) when row_lds,
// else from the block table.  qs: the scaled mean query (LDS).  Blocks j >= jk
// take their score from known[j] instead (blocks whose centroid another
// workgroup recomputed in the same launch: their fresh row may not be visible
// here, the score stored beside it with an agent-scope store is).  KNOWN_LDS:
// known[j - jk] is in this workgroup's LDS (it recomputed them itself).
template <int D, bool KNOWN_LDS = false>
__device__ __forceinline__ void rescore(const sel::SelectArgs &a, int b, int g,
                                        const int32_t *map, int m, const int *pages,
                                        bool row_lds, const float *qs, float *sc,
                                        const float *known, int jk) {
    constexpr int LPR = 16, VPL = D / LPR, RPI = kWave / LPR;
    constexpr int KU = 4, ROWS = kWaves * RPI * KU;  // 64 rows per pass
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int col = lane % LPR, rsub = lane / LPR;
    const int32_t *bt = a.bt + (size_t)b * a.max_blocks;
    float qf[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) qf[e] = qs[col * VPL + e];
    typedef floatx4_t Row[VPL / 4];
    struct Stage {
        Row cv[KU];
        int pg[KU], jj[KU];
        float kn[KU];
    };
    // two stages of ROWS rows in flight: the page ids come from LDS (or the
    // block table), then every row of the stage is requested at once
    auto issue = [&](Stage &st, int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = min(base + u * kWaves * RPI + wave * RPI + rsub, m - 1);
            st.jj[u] = map[row];
            st.pg[u] = row_lds ? pages[st.jj[u]] : bt[st.jj[u]];
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int p = st.pg[u] >= 0 && st.pg[u] < a.num_pages ? st.pg[u] : 0;
            const floatx4_t *src = reinterpret_cast<const floatx4_t *>(
                a.cent + ((size_t)p * a.Hkv + g) * D + col * VPL);
#pragma unroll
            for (int v = 0; v < VPL / 4; ++v) st.cv[u][v] = src[v];
            if constexpr (KNOWN_LDS)
                st.kn[u] = 0.f;  // read from LDS when the row is reduced
            else
                st.kn[u] = load_relaxed(known + min(st.jj[u], jk));
        }
    };
    auto reduce = [&](const Stage &st, int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = base + u * kWaves * RPI + wave * RPI + rsub;
            const float s = sel::row16_sum(sel::row_partial<VPL>(qf, st.cv[u]));
            const bool ok = st.pg[u] >= 0 && st.pg[u] < a.num_pages;
            if (col == 0 && row < m) {
                const float kn = KNOWN_LDS ? (st.jj[u] >= jk ? known[st.jj[u] - jk] : 0.f)
                                           : st.kn[u];
                sc[row] = !ok ? -INFINITY : st.jj[u] >= jk ? kn : s;
                if (!ok) flag_error(a.err, kErrPage);
            }
        }
    };
    if (m > 0) {
        Stage sa_, sb_;
        issue(sa_, 0);
        for (int base = 0;;) {
            if (base + ROWS < m) issue(sb_, base + ROWS);
            reduce(sa_, base);
            base += ROWS;
            if (base >= m) break;
            if (base + ROWS < m) issue(sa_, base + ROWS);
            reduce(sb_, base);
            base += ROWS;
            if (base >= m) break;
        }
    }
}

}  // namespace skt
}  // namespace btk
