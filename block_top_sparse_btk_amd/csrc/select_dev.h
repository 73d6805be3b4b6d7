// Device code of S2 + S3 (group scoring and top-k selection), shared by the
// stand-alone select kernel and the single-launch decode step.
// (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What carries
// the argument": key blocks are scored by their averaged key vectors per query
// group and the top k blocks are retrieved.)
//
// Scoring is a bandwidth-bound GEMV: a unit (sequence b, KV head g) streams the
// n_b centroid rows (D fp32 = 512 B at D=128) named by its block table.  The
// unit's blocks are cut into chunks; one 256-thread workgroup scores one chunk.
// The r query heads of the group are folded into their mean on entry
// (linearity: the mean of the heads' logits equals the logit of the mean query),
// so each block costs one D-long dot product.  16 lanes (one DPP row) hold a
// centroid row; loads run in two stages of KU rows per lane so one stage is in
// flight while the other is reduced (the stand-alone kernel takes KU = 4 to stay
// at five waves per SIMD, the decode step, whose attention already sets two
// waves per SIMD, KU = 8); scores are staged in LDS and leave the workgroup as
// contiguous stores.
//
// Selection runs in the workgroup that finishes a unit's last chunk (a counter
// per unit, see arrive_last), so it overlaps the scoring of later units.
#pragma once
#include "centroid_dev.h"

namespace btk {
namespace skt {
// A block sketch row's header (the layout and the rows are described with the
// sketch code, sketch_dev.h): the page the row was built from + 1 (0: none) and
// the scale of its codes.
struct SketchHdr {
    int32_t page1;
    float scale;
};
}  // namespace skt

namespace sel {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunk = 512;

struct SelectArgs {
    const void *q;
    const float *cent;
    const int32_t *bt;
    const int32_t *seq_lens;
    int32_t *indices;
    float *scores;
    uint32_t *counters;  // unit u's arrival counter at counters[u * kStateStride]
    uint32_t *err;
    int Hq, Hkv, num_pages, max_blocks, top_k, chunk, nchunk_max;
    float scale;
    // single-launch decode step only (NULL in the stand-alone select): the
    // chunk that holds a touched page recomputes its centroid (S1) first
    const void *k_cache;
    const int32_t *first_pos;
    float *cent_out;
    // shared-prefix form only (NULL otherwise): per (group, KV head) u = group *
    // Hkv + head, at pflags[u * kStateStride] and the word after it, the shared
    // items done and the members that have finished with them
    uint32_t *pflags = nullptr;
    // decode step with the KV append (NULL otherwise): the newest token's key
    // and value [B][Hkv][D] (the segment that refreshes that block averages the
    // key from here; the unit's attention item writes both into their cache
    // slot, position L - 1) and the caches they are written to
    const void *k_new = nullptr, *v_new = nullptr;
    void *k_out = nullptr, *v_out = nullptr;
    // decode step keeping block sketches current (NULL otherwise): the touched
    // blocks' sketch rows are rebuilt from their recomputed centroids
    skt::SketchHdr *sk_hdr = nullptr;
    uint8_t *sk_codes = nullptr;
};

// LDS used by one chunk's scan.
struct ScoreSmem {
    float *qraw;  // [r * D] the group's queries
    float *qs;    // [D] scaled mean query
    int *pages;   // [kMaxChunk] page ids of the chunk
    float *sc;    // [kMaxChunk] scores of the chunk
    int *flag;    // one word
    // decode step with the KV append: the new token's key row of the segment's
    // unit (D elements), loaded with the segment's setup
    uint32_t *newtok = nullptr;
};

// LDS used by the top-k selection.
// Radix histogram: 256 bins, then one spare bin per lane for keys out of range.
constexpr int kHistWords = 256 + kWave;
// The workgroup selection gives each of its (at most four) passes a histogram.
constexpr int kTopkPasses = 4;

struct TopkSmem {
    uint32_t *hist;      // [kTopkPasses * kHistWords] radix histograms
    uint32_t *cand;      // [256] compacted candidates
    uint32_t *red;       // [2 * kWaves]
    int *scan_red;       // [kWaves]
    uint32_t *keys;      // bitmaps of more than 2048 blocks: [16 * KMAX] words
};

// Where a selection goes: the caller's index row (or NULL) and, inside a
// decode step, the entries [lo, hi) of it into LDS for the workgroup's own
// attention (lds[i - lo] holds entry i; lo = hi = 0 when there is none).
// Pointers into LDS are never tested against NULL here: the compiler folded
// such a test into an operand form that gfx950 does not encode.
struct TopkOut {
    int32_t *idx;            // [top_k] or NULL
    int32_t *lds = nullptr;  // [hi - lo] or NULL
    int lo = 0, hi = 0;
    // the keys were a subset of the blocks, in ascending block order: key i is
    // block map[i] (LDS) when mapped, else block i
    const int32_t *map = nullptr;
    bool mapped = false;
    __device__ __forceinline__ void put(int pos, int32_t j) const {
        if (mapped && j >= 0) j = map[j];
        if (idx) store_relaxed_i32(idx + pos, j);
        if (pos >= lo && pos < hi) lds[pos - lo] = j;
    }
};

// Where the selecting workgroup reads a unit's scores from: fill() loads the
// float bits of blocks j = i * stride + first (0 for j >= nb), all loads in
// flight together.  The scores were stored by every chunk with store_relaxed
// before it counted itself in (see arrive_last).
struct PlainScores {
    const float *sc;  // [nb]
    template <int N>
    __device__ __forceinline__ void fill(uint32_t (&bits)[N], int first, int stride, int nb) const {
#pragma unroll
        for (int i = 0; i < N; ++i)  // unconditional (clamped): all in flight together
            bits[i] = __float_as_uint(load_relaxed(sc + min(i * stride + first, nb - 1)));
#pragma unroll
        for (int i = 0; i < N; ++i) bits[i] = i * stride + first < nb ? bits[i] : 0u;
    }
};

template <typename T>
__device__ __forceinline__ float load_q(const T *p);
template <>
__device__ __forceinline__ float load_q<uint16_t>(const uint16_t *p) {
    return bf16_bits_to_f32(*p);
}
template <>
__device__ __forceinline__ float load_q<float>(const float *p) {
    return *p;
}

// Sum of one wave-uniform count per wave over the workgroup (one barrier).
__device__ __forceinline__ int wg_sum(int wave_count, int *red, int &parity) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) red[parity * kWaves + wave] = wave_count;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[parity * kWaves + w];
    parity ^= 1;
    return s;
}

// Exclusive prefix sum over the workgroup in thread order.
__device__ __forceinline__ int wg_exclusive_scan(int x, int *red) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    __syncthreads();  // red may still be read by a previous step
    if (lane == kWave - 1) red[wave] = inc;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        if (w < wave) before += red[w];
    return before + inc - x;
}

// Wave-wide sum and max of a per-lane value, uniform result: DPP within each
// 16-lane row, then the four row results are read out.
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
    x += (uint32_t)dpp<0xB1>((int)x);   // quad xor 1
    x += (uint32_t)dpp<0x4E>((int)x);   // quad xor 2
    x += (uint32_t)dpp<0x141>((int)x);  // half-row mirror
    x += (uint32_t)dpp<0x140>((int)x);  // row mirror
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 0) + (uint32_t)__builtin_amdgcn_readlane((int)x, 16) +
           (uint32_t)__builtin_amdgcn_readlane((int)x, 32) + (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)dpp<0xB1>((int)x));
    x = max(x, (uint32_t)dpp<0x4E>((int)x));
    x = max(x, (uint32_t)dpp<0x141>((int)x));
    x = max(x, (uint32_t)dpp<0x140>((int)x));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}

// Wave-wide inclusive prefix sum (lane order) of a per-lane count, in DPP:
// shifts by 1, 2, 4, 8 within each 16-lane row, then the row totals are carried
// across rows with the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)dpp<0x111>((int)x);  // row_shr:1
    x += (uint32_t)dpp<0x112>((int)x);  // row_shr:2
    x += (uint32_t)dpp<0x114>((int)x);  // row_shr:4
    x += (uint32_t)dpp<0x118>((int)x);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// One radix-selection pass over the keys inside [lo, hi] (see select_topk_wave):
// histogram into 256 LDS bins of width 2^shift, locate the bin that holds the
// key of rank `need` counted from the top, and shrink [lo, hi] to it.  Keys out
// of range are counted in a per-lane spare bin, so the loop has no branches.
// The bin (of the 256 in hist) that holds the key of rank `need` counted from
// the top; `need` becomes that key's rank inside the bin and, if asked for,
// *count the number of keys in the bin.  Wave-uniform.
__device__ __forceinline__ uint32_t locate_bin(const uint32_t *hist, int &need, int lane,
                                               uint32_t *count = nullptr) {
    const u32x4_t h = reinterpret_cast<const u32x4_t *>(hist)[lane];  // bins 4l .. 4l+3
    const uint32_t lane_sum = h[0] + h[1] + h[2] + h[3];
    const uint32_t above_lane = wave_sum_u32(lane_sum) - wave_inclusive_scan(lane_sum);
    int bin = -1;
    uint32_t above_bin = 0u, in_bin = 0u, acc = above_lane;
    const uint32_t hv[4] = {h[0], h[1], h[2], h[3]};
#pragma unroll
    for (int e = 3; e >= 0; --e) {  // from this lane's top bin down
        if (bin < 0 && acc < (uint32_t)need && acc + hv[e] >= (uint32_t)need) {
            bin = 4 * lane + e;
            above_bin = acc;
            in_bin = hv[e];
        }
        acc += hv[e];
    }
    const int src = (int)__builtin_ctzll(__ballot(bin >= 0));  // exactly one lane has it
    need -= __builtin_amdgcn_readlane((int)above_bin, src);
    if (count) *count = (uint32_t)__builtin_amdgcn_readlane((int)in_bin, src);
    return (uint32_t)__builtin_amdgcn_readlane(bin, src);
}

template <int N>
__device__ __forceinline__ void radix_pass(const uint32_t (&key)[N], uint32_t &lo, uint32_t &hi,
                                           int &need, uint32_t *hist, int lane) {
    const uint32_t span = hi - lo;
    const int shift = max(0, 24 - __builtin_clz(span));  // (span >> shift) < 256
    reinterpret_cast<u32x4_t *>(hist)[lane] = u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t off = key[i] - lo;
        atomicAdd(&hist[off <= span ? (off >> shift) : 256u + lane], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    const uint32_t b_sel = locate_bin(hist, need, lane);
    const uint32_t top = (b_sel << shift) + ((1u << shift) - 1u);  // bin's top offset
    if (top < span) hi = lo + top;
    lo += b_sel << shift;
}

// Number of the wave's keys inside [lo, hi] (wave-uniform).
template <int N>
__device__ __forceinline__ int count_in_range(const uint32_t (&key)[N], uint32_t lo, uint32_t hi) {
    int m = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) m += __popcll(__ballot(key[i] - lo <= hi - lo));
    return m;
}

// Writes the wave's keys inside [lo, hi] to cand[0 .. m), slot by slot.
template <int N>
__device__ __forceinline__ void compact(const uint32_t (&key)[N], uint32_t lo, uint32_t hi,
                                        uint32_t *cand, int lane) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const bool in = key[i] - lo <= hi - lo;
        const uint64_t mask = __ballot(in);
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                   (uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (in) cand[pos] = key[i];
        base += __popcll(mask);
    }
}

// The end of a radix selection, by one wave: the m <= 256 keys still inside
// [lo, hi] are in cand[0 .. m).  They are taken four per lane for cheap passes;
// once at most 64 are left each lane counts the candidates above and at its own
// key, which names T directly.  On return lo = T and need = the number of keys
// equal to T to keep.  Uses cand and hist.
__device__ __forceinline__ void finish_from_cand(uint32_t *cand, int m, uint32_t &lo, uint32_t &hi,
                                                 int &need, uint32_t *hist, int lane) {
    uint32_t k4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) k4[e] = e * kWave + lane < m ? cand[e * kWave + lane] : 0u;
    __builtin_amdgcn_wave_barrier();
    cand[lane] = 0u;  // the finisher reads all 64 slots: absent keys are 0
    __builtin_amdgcn_wave_barrier();
    while (lo < hi && m > kWave) {
        radix_pass(k4, lo, hi, need, hist, lane);
        m = count_in_range(k4, lo, hi);
    }
    if (lo < hi) {
        // at most 64 keys left: every lane ranks its own against all of them
        // (LDS broadcast reads); T is the one of rank `need`
        compact(k4, lo, hi, cand, lane);
        __builtin_amdgcn_wave_barrier();
        // all 64 slots at once (slots from m on hold 0, below every key)
        const uint32_t mine = lane < m ? cand[lane] : 0u;
        u32x4_t c4[kWave / 4];
#pragma unroll
        for (int t = 0; t < kWave / 4; ++t) c4[t] = reinterpret_cast<const u32x4_t *>(cand)[t];
        int gt = 0, ge = 0;
#pragma unroll
        for (int t = 0; t < kWave / 4; ++t) {
            const uint32_t cv[4] = {c4[t][0], c4[t][1], c4[t][2], c4[t][3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gt += cv[e] > mine ? 1 : 0;
                ge += cv[e] >= mine ? 1 : 0;
            }
        }
        const int src_lane = (int)__builtin_ctzll(__ballot(lane < m && gt < need && ge >= need));
        lo = (uint32_t)__builtin_amdgcn_readlane((int)mine, src_lane);
        need -= __builtin_amdgcn_readlane(gt, src_lane);  // keys equal to T to take
    }
}

// Writes the winners in ascending block order, by one wave: lane l holds the
// NW bitmap words a[w] (keys above T) and e[w] (keys equal to T) of blocks
// [32 (NW l + w), 32 (NW l + w) + 32); every key above T is kept, then keys
// equal to T in block order until take_eq.
template <int NW>
__device__ __forceinline__ void write_winners(uint32_t (&a)[NW], uint32_t (&e)[NW], int take_eq,
                                              int kb, int top_k, const TopkOut &out, int lane) {
    uint32_t ecnt = 0u, acnt = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) ecnt += (uint32_t)__popc(e[w]);
    int e_before = (int)(wave_inclusive_scan(ecnt) - ecnt);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        while (e[w] && e_before < take_eq) {  // lowest-index equal keys first
            const uint32_t bit = e[w] & (0u - e[w]);
            a[w] |= bit;
            e[w] ^= bit;
            ++e_before;
        }
        acnt += (uint32_t)__popc(a[w]);
    }
    int pos = (int)(wave_inclusive_scan(acnt) - acnt);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        while (a[w]) {
            if (pos < kb) out.put(pos, (NW * lane + w) * 32 + __builtin_ctz(a[w]));
            ++pos;
            a[w] &= a[w] - 1u;
        }
    }
    for (int i = kb + lane; i < top_k; i += kWave) out.put(i, -1);
}

// Top-k of a unit's nb scores in one wave (nb <= 64 * KMAX <= 2048).
// Lane l holds the keys of blocks i*64 + l in registers.  The kb-th largest key
// T is found by radix selection over value ranges: a pass histograms the keys
// inside [lo, hi] into 256 bins and shrinks [lo, hi] to the bin holding the rank
// still needed, resolving eight bits.  The first pass leaves about a hundred
// keys in range at the usual score spreads (its top bins span whole binades):
// up to 256 are compacted and finished by finish_from_cand.  The winners
// (every key above T, then keys equal to T in block order until kb) are
// recorded as bitmaps built from ballots (slot i's ballot covers words 2i and
// 2i+1) and a popcount prefix sum writes them in ascending block order.
template <int KMAX, typename Src>
__device__ __forceinline__ void select_topk_wave(const Src &src, int nb, int top_k,
                                                 const TopkOut &out, TopkSmem &sm) {
    static_assert(KMAX <= 32, "one bitmap word per lane covers 2048 blocks");
    uint32_t *hist = sm.hist, *cand = sm.cand;
    const int lane = threadIdx.x & (kWave - 1);
    const int kb = min(top_k, nb);
    uint32_t key[KMAX];
    src.fill(key, lane, kWave, nb);
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int j = i * kWave + lane;
        key[i] = j < nb ? score_key(__uint_as_float(key[i])) : 0u;  // 0 = no key
        kmin = j < nb ? min(kmin, key[i]) : kmin;
        kmax = max(kmax, key[i]);
    }
    uint32_t lo = ~wave_max_u32(~kmin), hi = wave_max_u32(kmax);
    int need = kb;  // rank of T among the keys inside [lo, hi], counted from the top
    if (lo < hi) radix_pass(key, lo, hi, need, hist, lane);
    if (lo < hi) {
        int m = count_in_range(key, lo, hi);
        while (lo < hi && m > 4 * kWave) {  // rare: keys bunched in one bin
            radix_pass(key, lo, hi, need, hist, lane);
            m = count_in_range(key, lo, hi);
        }
        if (lo < hi) {
            compact(key, lo, hi, cand, lane);
            __builtin_amdgcn_wave_barrier();
            finish_from_cand(cand, m, lo, hi, need, hist, lane);
        }
    }
    const uint32_t T = lo;
    // bitmaps: lane l's words cover blocks [32l, 32l + 32), the low or high
    // half of slot l/2's ballot (lanes from 2*KMAX on hold none)
    uint32_t a[1] = {0u}, e[1] = {0u};
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const uint64_t ab = __ballot(key[i] > T);
        const uint64_t eb = __ballot(key[i] == T);  // absent keys are 0 < T
        if ((lane >> 1) == i) {
            a[0] = (lane & 1) ? (uint32_t)(ab >> 32) : (uint32_t)ab;
            e[0] = (lane & 1) ? (uint32_t)(eb >> 32) : (uint32_t)eb;
        }
    }
    write_winners<1>(a, e, need, kb, top_k, out, lane);
}

// Top-k of a unit's nb <= 256 * KMAX <= 8192 scores by the four waves of the
// workgroup.  Thread t holds the keys of blocks i*256 + t.  The radix passes of
// select_topk_wave run over the workgroup, each into its own LDS histogram (all
// of them cleared while the keys are in flight), so that a pass costs a single
// barrier: every wave then locates the bin itself (identical results).  Each
// pass resolves eight bits of the range, so at most four reach lo = hi = T; a
// pass whose bin is taken whole ends the search early (T just below the bin,
// no equal keys to take), which usually happens by the second.
// The first range starts at a lower bound of T rather than at the smallest key:
// for kb <= 64, the smallest of the largest keys of a wave's first kb lanes
// (kb keys lie at or above it), the largest of these over the waves.  Bitmaps
// come from per-wave ballots: slot i of wave v covers blocks 256i + 64v .. +63,
// words 8i + 2v and 8i + 2v + 1; they are gathered in LDS (cand up to 2048
// blocks, the key area beyond) and wave 0 writes the winners, KMAX / 8 words
// per lane.
template <int KMAX, typename Src>
__device__ __forceinline__ void select_topk_wg4(const Src &src, int nb, int top_k,
                                                const TopkOut &out, TopkSmem &sm) {
    static_assert(KMAX == 4 || KMAX == 8 || KMAX == 16 || KMAX == 32, "8 KMAX bitmap words");
    constexpr int NW = KMAX <= 8 ? 1 : KMAX / 8;  // bitmap words per lane of wave 0
    constexpr int NWORDS = 8 * KMAX;
    uint32_t *red = sm.red;
    uint32_t *bm = KMAX <= 8 ? sm.cand : sm.keys;  // [0, NWORDS) above T, then equal
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int kb = min(top_k, nb);
    for (int i = tid; i < kTopkPasses * kHistWords / 4; i += kThreads)
        reinterpret_cast<u32x4_t *>(sm.hist)[i] = u32x4_t{0u, 0u, 0u, 0u};
    uint32_t key[KMAX];
    src.fill(key, tid, kThreads, nb);
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int j = i * kThreads + tid;
        key[i] = j < nb ? score_key(__uint_as_float(key[i])) : 0u;  // 0 = no key
        kmin = j < nb ? min(kmin, key[i]) : kmin;
        kmax = max(kmax, key[i]);
    }
    // nb > 256: every thread holds at least one key, so kmax is a key
    const uint32_t bound = kb <= kWave ? (lane < kb ? kmax : 0xffffffffu) : kmin;
    const uint32_t wave_lo = ~wave_max_u32(~bound);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
        red[wave] = wave_lo;
        red[kWaves + wave] = kmax;
    }
    __syncthreads();  // also orders the histogram clears before the passes
    uint32_t lo = kb <= kWave ? max(max(red[0], red[1]), max(red[2], red[3]))
                              : min(min(red[0], red[1]), min(red[2], red[3]));
    uint32_t hi = max(max(red[kWaves], red[kWaves + 1]), max(red[kWaves + 2], red[kWaves + 3]));
    int need = kb;  // rank of T among the keys inside [lo, hi], counted from the top
#pragma unroll 1
    for (int p = 0; p < kTopkPasses && lo < hi; ++p) {
        uint32_t *hist = sm.hist + p * kHistWords;
        const uint32_t span = hi - lo;
        const int shift = max(0, 24 - __builtin_clz(span));  // (span >> shift) < 256
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
            const uint32_t off = key[i] - lo;
            atomicAdd(&hist[off <= span ? (off >> shift) : 256u + lane], 1u);
        }
        __syncthreads();
        uint32_t in_bin;
        const uint32_t b_sel = locate_bin(hist, need, lane, &in_bin);  // every wave, same result
        const uint32_t top = (b_sel << shift) + ((1u << shift) - 1u);
        if (top < span) hi = lo + top;
        lo += b_sel << shift;
        if (in_bin == (uint32_t)need && lo < hi) {  // every key of the bin is kept
            hi = --lo;  // lo >= 1: valid keys are nonzero
            need = 0;
        }
    }
    const uint32_t T = lo;  // need: the keys equal to T to keep
    // bitmaps through LDS: above in bm[0 .. NWORDS), equal in bm[NWORDS .. 2 NWORDS)
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const uint64_t ab = __ballot(key[i] > T);
        const uint64_t eb = __ballot(key[i] == T);  // absent keys are 0 < T
        if (lane == 0) {
            bm[8 * i + 2 * wave] = (uint32_t)ab;
            bm[8 * i + 2 * wave + 1] = (uint32_t)(ab >> 32);
            bm[NWORDS + 8 * i + 2 * wave] = (uint32_t)eb;
            bm[NWORDS + 8 * i + 2 * wave + 1] = (uint32_t)(eb >> 32);
        }
    }
    __syncthreads();
    if (wave == 0) {
        uint32_t a[NW], e[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int word = NW * lane + w;
            a[w] = word < NWORDS ? bm[word] : 0u;
            e[w] = word < NWORDS ? bm[NWORDS + word] : 0u;
        }
        write_winners<NW>(a, e, need, kb, top_k, out, lane);
    }
}

// Selection of a unit's top-k blocks by a whole workgroup: one wave up to 256
// blocks (no barrier), the four waves beyond (radix passes, a histogram each;
// the bitmaps of more than 2048 blocks go through the key area of TopkSmem,
// which then holds at least 16 * KMAX words).
template <typename Src>
__device__ __forceinline__ void select_topk(const Src &src, int nb, int top_k,
                                            const TopkOut &out, TopkSmem &sm) {
    const int tid = threadIdx.x;
    if (min(top_k, nb) == nb) {  // every block is kept
        for (int i = tid; i < top_k; i += kThreads) out.put(i, i < nb ? i : -1);
        return;
    }
    if (nb > 4 * kWave) {  // the whole workgroup, up to 32 keys per thread
        if (nb <= 4 * kThreads) select_topk_wg4<4>(src, nb, top_k, out, sm);
        else if (nb <= 8 * kThreads) select_topk_wg4<8>(src, nb, top_k, out, sm);
        else if (nb <= 16 * kThreads) select_topk_wg4<16>(src, nb, top_k, out, sm);
        else select_topk_wg4<32>(src, nb, top_k, out, sm);
        return;
    }
    if (tid >= kWave) return;
    select_topk_wave<4>(src, nb, top_k, out, sm);
}

// Sum over the 16 lanes of a DPP row (result in every lane of the row).
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0xB1, 0xF, 0xF, false));  // quad xor 1
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x4E, 0xF, 0xF, false));  // quad xor 2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x141, 0xF, 0xF, false));  // half mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x140, 0xF, 0xF, false));  // mirror
    return x;
}

// The per-lane part of a centroid row's dot product with the scaled mean
// query (VPL floats per lane).  Every scoring path (the scan, the shared-prefix
// rows, the decode step's re-score of a freshly updated centroid) shares it,
// and its operations are fixed (per four floats one product, then three fused
// multiply-adds, then one add; no contraction) so that every kernel computes
// bit-identical scores whatever its code generation.
template <int VPL>
__device__ __forceinline__ float row_partial(const float (&qf)[VPL], const floatx4_t (&cv)[VPL / 4]) {
#pragma clang fp contract(off)
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < VPL / 4; ++v) {
        float t = qf[4 * v] * cv[v][0];
        t = __builtin_fmaf(qf[4 * v + 1], cv[v][1], t);
        t = __builtin_fmaf(qf[4 * v + 2], cv[v][2], t);
        t = __builtin_fmaf(qf[4 * v + 3], cv[v][3], t);
        s = s + t;
    }
    return s;
}

// The setup loads of a chunk or segment in one round trip: the group's r
// queries into sm.qraw and n (<= PMAX) page ids of sequence b's block-table row
// from block j0 into sm.pages.  Every load is unconditional (addresses clamped
// into range, surplus results dropped), because a conditional load compiles to
// a branch that waits for it before the next one is issued.
template <typename T, int D, int PMAX>
__device__ __forceinline__ void load_setup(const SelectArgs &a, int b, int g, int j0, int n,
                                           ScoreSmem &sm) {
    constexpr int QN = (kMaxGroup * D + kThreads - 1) / kThreads;
    constexpr int PN = (PMAX + kThreads - 1) / kThreads;
    const int tid = threadIdx.x, r = a.Hq / a.Hkv;
    const T *qp = static_cast<const T *>(a.q) + ((size_t)b * a.Hq + (size_t)g * r) * D;
    const int32_t *row = a.bt + (size_t)b * a.max_blocks + j0;
    float qv[QN];
    int32_t pv[PN];
#pragma unroll
    for (int k = 0; k < QN; ++k) qv[k] = load_q<T>(qp + min(k * kThreads + tid, r * D - 1));
    if (n > 0) {
#pragma unroll
        for (int k = 0; k < PN; ++k) pv[k] = row[min(k * kThreads + tid, n - 1)];
    }
#pragma unroll
    for (int k = 0; k < QN; ++k)
        if (k * kThreads + tid < r * D) sm.qraw[k * kThreads + tid] = qv[k];
    if (n > 0) {
#pragma unroll
        for (int k = 0; k < PN; ++k)
            if (k * kThreads + tid < n) sm.pages[k * kThreads + tid] = pv[k];
    }
}

// Scores n consecutive blocks j0 .. j0+n-1 of unit (b, g) whose page ids are in
// sm.pages[0 .. n) (invalid ones as -1) against the scaled mean query in
// sm.qs, stages the scores in sm.sc and stores them to a.scores.  REFRESH
// (the decode step, a.first_pos set): the pages touched since the last step
// also get their centroid recomputed from the keys, stored for later steps and
// re-scored here.  KU: rows per lane per pipeline stage (two stages of
// 4 * 4 * KU rows are in flight).  Called with sm.pages and sm.qs visible to
// every thread; ends with the stores issued (not waited for).
}  // namespace sel

namespace skt {
// Writes sketch row `row` from a centroid of which this lane holds dims
// lane * E .. lane * E + E - 1 (E = D / 64), page id `page` (wave-uniform call).
template <int D>
__device__ __forceinline__ void encode_row(const float (&x)[D / kWave], int page, size_t row,
                                           SketchHdr *hdr, uint8_t *codes, int lane) {
    constexpr int E = D / kWave;
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) m = max(m, __float_as_uint(fabsf(x[e])));
    const float amax = __uint_as_float(sel::wave_max_u32(m));
    const float scale = amax / 127.0f;
    uint32_t packed = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        float qv = amax > 0.f ? rintf(x[e] / scale) : 0.f;
        qv = fminf(fmaxf(qv, -127.f), 127.f);
        packed |= (uint32_t)((int)qv + 128) << (8 * e);
    }
    uint8_t *dst = codes + row * D + lane * E;
    if constexpr (E == 2)
        *reinterpret_cast<uint16_t *>(dst) = (uint16_t)packed;
    else
        *dst = (uint8_t)packed;
    if (lane == 0) hdr[row] = SketchHdr{page + 1, scale};
}
}  // namespace skt

namespace sel {

template <typename T, int D, int KU, bool REFRESH, bool APPEND = false>
__device__ __forceinline__ void scan_rows(const SelectArgs &a, int b, int g, int j0, int n, int L,
                                          int fp, ScoreSmem &sm, float *crow) {
    constexpr int LPR = 16;                       // lanes per centroid row: one DPP row
    constexpr int VPL = D / LPR;                  // floats per lane per row (8 or 4)
    constexpr int RPI = kWave / LPR;              // rows per wave per load step
    constexpr int ROWS = kWaves * RPI * KU;       // rows per workgroup stage
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int col = lane % LPR, rsub = lane / LPR;
    // decode step: wave w refreshes the touched blocks jw, jw + 4, ... of the
    // run; the keys of its first one are requested before the scan so that
    // they arrive while it streams
    const bool refresh = REFRESH && (a.first_pos || APPEND) && fp >= 0 && fp < L;
    const int jw = refresh ? max(j0, fp / kPage) + wave : j0 + n;
    const T *keys = static_cast<const T *>(a.k_cache) + (size_t)g * kPage * D;
    const size_t page_stride = (size_t)a.Hkv * kPage * D;
    KeyTile<T, D> kt;
    // with the KV append the newest token (position L - 1) is the last of its
    // block and is never read from the cache: it comes from k_new
    const int jnew = APPEND ? (L - 1) / kPage : -1;
    auto cached = [&](int j) { return min(kPage, L - j * kPage) - (j == jnew ? 1 : 0); };
    if (jw < j0 + n && sm.pages[jw - j0] >= 0)
        kt.load(keys + (size_t)sm.pages[jw - j0] * page_stride, cached(jw), lane);
    float qf[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) qf[e] = sm.qs[col * VPL + e];
    // Loads are unconditional so that the next stage stays in flight while the
    // current one is reduced: rows past the run re-read its last row and an
    // invalid page reads page 0; neither result is kept.
    typedef floatx4_t Row[VPL / 4];
    auto issue = [&](Row (&cv)[KU], int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = min(base + u * kWaves * RPI + wave * RPI + rsub, n - 1);
            const int p = max(sm.pages[row], 0);
            const floatx4_t *src = reinterpret_cast<const floatx4_t *>(
                a.cent + ((size_t)p * a.Hkv + g) * D + col * VPL);
#pragma unroll
            for (int v = 0; v < VPL / 4; ++v) cv[u][v] = src[v];
        }
    };
    auto reduce = [&](const Row (&cv)[KU], int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = base + u * kWaves * RPI + wave * RPI + rsub;
            const float s = row16_sum(row_partial<VPL>(qf, cv[u]));
            if (col == 0 && row < n) sm.sc[row] = sm.pages[row] >= 0 ? s : -INFINITY;
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

    // decode step: the touched blocks' centroids are recomputed, stored for
    // later steps and re-scored (crow is the wave's LDS row).  The scan's own
    // score of a touched block comes from another wave: it must land first.
    if (refresh && max(j0, fp / kPage) < j0 + n) __syncthreads();
    for (int j = jw; j < j0 + n; j += kWaves) {
        const int page = sm.pages[j - j0];
        if (page < 0) continue;
        const int v = min(kPage, L - j * kPage);
        float *row_lds = crow + wave * D;
        if (j != jw) kt.load(keys + (size_t)page * page_stride, cached(j), lane);
        if (APPEND && j == jnew)  // this lane's 16-byte slice of the new key (LDS)
            kt.set_row(v - 1,
                       *reinterpret_cast<const u32x4_t *>(sm.newtok + (lane % KeyTile<T, D>::LPR) *
                                                        (KeyTile<T, D>::VEC * sizeof(T) / 4)),
                       lane);
        kt.mean_to(v, a.cent_out + ((size_t)page * a.Hkv + g) * D, row_lds, true, lane);
        __builtin_amdgcn_wave_barrier();
        Row cv;
#pragma unroll
        for (int vv = 0; vv < VPL / 4; ++vv)
            cv[vv] = reinterpret_cast<const floatx4_t *>(row_lds + col * VPL)[vv];
        const float s = row16_sum(row_partial<VPL>(qf, cv));
        if (lane == 0) sm.sc[j - j0] = s;
        if (a.sk_hdr) {  // the block's sketch row, from the same centroid
            constexpr int E = D / kWave;
            float x[E];
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = row_lds[lane * E + e];
            skt::encode_row<D>(x, page, ((size_t)b * a.Hkv + g) * a.max_blocks + j, a.sk_hdr,
                               a.sk_codes, lane);
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    float *sc = a.scores + ((size_t)b * a.Hkv + g) * a.max_blocks;
    for (int i = tid; i < n; i += kThreads) store_relaxed(sc + j0 + i, sm.sc[i]);
}

// Marks the n page ids in sm.pages that are out of range as -1 (error bit).
__device__ __forceinline__ void check_pages(const SelectArgs &a, ScoreSmem &sm, int n) {
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int p = sm.pages[i];
        if (p < 0 || p >= a.num_pages) {
            flag_error(a.err, kErrPage);
            sm.pages[i] = -1;
        }
    }
}

// The group's mean query, pre-scaled, from the r raw queries in sm.qraw.
template <int D>
__device__ __forceinline__ void mean_query(const SelectArgs &a, ScoreSmem &sm) {
    const int r = a.Hq / a.Hkv;
    if (threadIdx.x < D) {
        float s = 0.f;
        for (int h = 0; h < r; ++h) s += sm.qraw[h * D + threadIdx.x];
        sm.qs[threadIdx.x] = s * (a.scale / (float)r);
    }
}

// Scores one chunk of a unit's blocks into a.scores (and, inside a decode step,
// first refreshes the centroids of the chunk's touched pages).  Returns true in
// the workgroup that completed the unit's last chunk, which must then select;
// nb receives the unit's block count (-1 for an invalid length, whose only
// chunk writes -1 indices).  skip: leading blocks scored elsewhere (a shared
// prompt prefix) by `extra` other workgroups that count in on the unit too; the
// chunks cover blocks [skip, n_b), and a unit with nothing left still has
// chunk 0, which only counts in.
template <typename T, int D, int KU>
__device__ __forceinline__ bool score_chunk(const SelectArgs &a, int unit, int c, ScoreSmem &sm,
                                            float *crow, int &nb_out, int skip = 0,
                                            int extra = 0) {
    const int tid = threadIdx.x;
    const int b = unit / a.Hkv, g = unit % a.Hkv;
    int32_t *out = a.indices + (size_t)unit * a.top_k;
    const int j0 = skip + c * a.chunk;

    // setup in one round trip: the group's queries, the chunk's slice of the
    // block-table row (entries past the sequence are read but never used), the
    // length and the decode position
    // (length and decode position requested after the rest, so that waiting
    // for them, as scalar values, waits for everything at once)
    load_setup<T, D, kMaxChunk>(a, b, g, j0, min(a.chunk, a.max_blocks - j0), sm);
    const int L = a.seq_lens[b];
    const int fp = a.first_pos ? a.first_pos[b] : -1;
    __syncthreads();

    if (L < 1 || L > a.max_blocks * kPage) {
        if (c == 0) {
            for (int i = tid; i < a.top_k; i += kThreads) store_relaxed_i32(out + i, -1);
            if (tid == 0) flag_error(a.err, kErrSeqLen);
        }
        nb_out = -1;  // an invalid length has exactly one item, chunk 0
        return false;
    }
    const int nb = (L + kPage - 1) / kPage;
    const int nchunks = max(1, (nb - skip + a.chunk - 1) / a.chunk);
    if (c >= nchunks) return false;
    const int n = max(0, min(nb, j0 + a.chunk) - j0);
    check_pages(a, sm, n);  // the entries this thread loaded
    mean_query<D>(a, sm);
    __syncthreads();
    scan_rows<T, D, KU, false>(a, b, g, j0, n, L, fp, sm, crow);
    nb_out = nb;
    return arrive_last(&a.counters[(size_t)unit * kStateStride], (uint32_t)(nchunks + extra),
                       sm.flag);
}

// Decode step: scores blocks [j0, j1) of unit (b, g) of a sequence of length L
// with decode position fp, in runs of up to RUN blocks (sm.pages and sm.sc hold
// RUN entries; a run costs one round trip for its page ids).  cont: the same
// workgroup scored this unit's blocks up to j0 just before, so the group's mean
// query is still in sm.qs and only page ids are loaded.  Ends with the score
// stores issued (not waited for); the caller counts the blocks in later (see
// count_in).
template <typename T, int D, int KU, int RUN, bool APPEND = false>
__device__ __forceinline__ void score_span(const SelectArgs &a, int b, int g, int j0, int j1,
                                           int L, int fp, bool cont, ScoreSmem &sm,
                                           float *crow) {
    const int tid = threadIdx.x;
    const int32_t *row = a.bt + (size_t)b * a.max_blocks;
    constexpr int PN = RUN / kThreads;
    auto load_pages = [&](int s0, int n) {  // all loads in flight together
        int32_t pv[PN];
#pragma unroll
        for (int k = 0; k < PN; ++k) pv[k] = row[s0 + min(k * kThreads + tid, n - 1)];
#pragma unroll
        for (int k = 0; k < PN; ++k)
            if (k * kThreads + tid < n) sm.pages[k * kThreads + tid] = pv[k];
    };
    int n = min(RUN, j1 - j0);
    // setup in one round trip: (the group's queries and) the first run's page ids
    if (cont) load_pages(j0, n);
    else load_setup<T, D, RUN>(a, b, g, j0, n, sm);
    if constexpr (APPEND) {  // the span that holds the newest token takes its key
        const int jn = (L - 1) / kPage;
        if (j0 <= jn && jn < j1) {
            constexpr int W = D * (int)sizeof(T) / 4;  // 32-bit words per row
            const uint32_t *kr = reinterpret_cast<const uint32_t *>(
                static_cast<const T *>(a.k_new) + ((size_t)b * a.Hkv + g) * D);
            for (int i = tid; i < W; i += kThreads) sm.newtok[i] = kr[i];
        }
    }
    __syncthreads();
    if (!cont) mean_query<D>(a, sm);
    for (int s0 = j0;;) {
        check_pages(a, sm, n);
        __syncthreads();
        scan_rows<T, D, KU, true, APPEND>(a, b, g, s0, n, L, fp, sm, crow);
        s0 += n;
        if (s0 >= j1) break;
        n = min(RUN, j1 - s0);
        __syncthreads();  // sm.pages and sm.sc are free again
        load_pages(s0, n);
    }
}

// Decode step: counts cnt freshly scored blocks of unit `unit` (nb blocks) in,
// once this workgroup's score stores have completed.  The count that completes
// the unit resets the counter and sets the unit's ready word to `tag`; every
// other workgroup's stores were complete before it counted in, so a reader
// that sees the tag sees every score.
__device__ __forceinline__ void count_in(const SelectArgs &a, int unit, int cnt, int nb,
                                         uint32_t *ready, uint32_t tag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *c = &a.counters[(size_t)unit * kStateStride];
        const uint32_t prev = __hip_atomic_fetch_add(c, (uint32_t)cnt, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev + (uint32_t)cnt == (uint32_t)nb) {
            __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ready, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Decode step: a unit whose length is invalid has a single placeholder row; it
// writes -1 indices, flags the error and marks the unit ready.
__device__ __forceinline__ void invalid_unit(const SelectArgs &a, int unit, uint32_t *ready,
                                             uint32_t tag) {
    const int tid = threadIdx.x;
    int32_t *out = a.indices + (size_t)unit * a.top_k;
    for (int i = tid; i < a.top_k; i += kThreads) store_relaxed_i32(out + i, -1);
    if (tid == 0) flag_error(a.err, kErrSeqLen);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(ready, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decode step: scores blocks [j0, j1) of unit (b, g) (a sequence of length L
// with nb blocks, decode position fp; nb < 0: an invalid length, whose single
// placeholder row writes -1 indices) and counts them in on the unit's counter;
// the segment that completes the unit sets its ready word to `tag`.
template <typename T, int D, int KU, int RUN, bool APPEND = false>
__device__ __forceinline__ void score_segment(const SelectArgs &a, int b, int g, int j0, int j1,
                                              int nb, int L, int fp, ScoreSmem &sm, float *crow,
                                              uint32_t *ready, uint32_t tag) {
    const int unit = b * a.Hkv + g;
    if (nb < 0) {
        invalid_unit(a, unit, ready, tag);
        return;
    }
    score_span<T, D, KU, RUN, APPEND>(a, b, g, j0, j1, L, fp, false, sm, crow);
    count_in(a, unit, j1 - j0, nb, ready, tag);
}

}  // namespace sel
}  // namespace btk
