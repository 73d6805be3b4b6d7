// Block sketches and the selection that uses them (S2 + S3 with the same
// result as btk_select).  (Pith review of "Kinetics: Rethinking Test-Time
// Scaling Laws", "What carries the argument": blocks are scored by their
// averaged keys and the k best are kept.  The sketch changes which centroid
// rows are read, not which blocks are selected.)
//
// A sketch row is an 8-bit copy of one block's fp32 centroid, kept per sequence
// in block-table order, so that a unit's sketch is one contiguous stream:
//   header[i] = {page + 1 (0: no sketch), scale = amax / 127}
//   codes[i][d] = rint(c_d / scale) + 128  (in 1 .. 255; 128 when amax = 0)
// for row i = (b * Hkv + g) * max_blocks + j (block j of sequence b, KV head g).
//
// Why the selection is unchanged.  With c the fp32 centroid, qs the scaled mean
// query and s = qs . c, the sketch gives sa = scale * (sum_d qs_d * code_d -
// 128 * sum_d qs_d).  Rounding c_d / scale to an integer moves each term by at
// most 0.50001 * scale * |qs_d| (the fp32 quotient is within 127 * 2^-24 of
// exact), and the fp32 evaluation of either sum, in any order, by at most
// 127 * 2^-24 * (255 + 128) * scale * |qs|_1 (the sketch's) and
// 127 * 2^-24 * 127 * scale * |qs|_1 (the exact score's), about 0.004 *
// scale * |qs|_1 together.  So every score s computed by the fp32 scan lies in
// [sa - e, sa + e] with e = 0.51 * scale * |qs|_1 (the margin also covers the
// rounding of sa - e and sa + e themselves).  With tau the kb-th largest lower
// end, at least kb blocks score at least tau; a block whose upper end is below
// tau therefore scores below kb others and cannot be selected under any tie
// rule.  The remaining candidates are scored exactly as btk_select scores them
// (the same code, the same bits) and the top kb of those are selected with the
// same tie rule, so the indices equal btk_select's.  A row whose header does
// not name the block's current page (not built, stale, invalid page) is always
// a candidate; when candidates exceed the LDS map every block is scored.
#include "select_dev.h"

namespace btk {
namespace {

using sel::kThreads;
using sel::kWaves;
using sel::kMaxChunk;

struct SketchHdr {
    int32_t page1;
    float scale;
};

constexpr float kBoundFactor = 0.51f;
constexpr int kCandCap = 2048;  // candidates whose block ids fit the LDS map

struct SketchArgs {
    const SketchHdr *hdr;   // [units * max_blocks]
    const uint8_t *codes;   // [units * max_blocks][D]
    float *lo, *hi;         // [units * max_blocks] interval ends (workspace)
    float *exact;           // [units * max_blocks] exact scores of candidates (workspace)
};

// ---- building the sketch -------------------------------------------------
//
// One wave per row: the centroid row is read (D / 64 floats per lane), its
// largest magnitude reduced over the wave, and the codes and header written.
// Workgroup (unit, chunk) covers blocks [c * per, (c + 1) * per) of the unit;
// with first_pos, blocks before first_pos[b] / 16 are left as they are.
template <int D>
__global__ __launch_bounds__(kThreads) void sketch_update_kernel(
    const float *__restrict__ cent, const int32_t *__restrict__ bt,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ first_pos, int Hkv,
    int max_blocks, int num_pages, int per, int nch, SketchHdr *__restrict__ hdr,
    uint8_t *__restrict__ codes, uint32_t *err) {
    constexpr int E = D / kWave;  // floats per lane
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int unit = blockIdx.x / nch, c = blockIdx.x % nch;
    const int b = unit / Hkv, g = unit % Hkv;
    const int L = seq_lens[b];
    if (L < 1 || L > max_blocks * kPage) {
        if (c == 0 && threadIdx.x == 0) flag_error(err, kErrSeqLen);
        return;
    }
    const int nb = (L + kPage - 1) / kPage;
    int j0 = c * per;
    if (first_pos) {
        const int fp = first_pos[b];
        j0 = max(j0, fp > 0 ? fp / kPage : 0);
    }
    const int j1 = min(nb, (c + 1) * per);
    for (int j = j0 + wave; j < j1; j += kWaves) {
        const size_t row = (size_t)unit * max_blocks + j;
        const int page = bt[(size_t)b * max_blocks + j];
        if (page < 0 || page >= num_pages) {
            if (lane == 0) {
                flag_error(err, kErrPage);
                hdr[row] = SketchHdr{0, 0.f};
            }
            continue;
        }
        const float *src = cent + ((size_t)page * Hkv + g) * D + lane * E;
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = src[e];
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
}

// ---- the selection ---------------------------------------------------------

// The kb-th largest of the nb keys of src (order-preserving score keys; 0 = no
// key), returned as a key tau such that at least kb keys are >= tau and every
// key above the kb-th largest is >= tau.  The radix passes of select_topk_wg4;
// every thread gets the result.
template <int KMAX, typename Src>
__device__ uint32_t kth_key_wg4(const Src &src, int nb, int kb, sel::TopkSmem &sm) {
    uint32_t *red = sm.red;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    for (int i = tid; i < sel::kTopkPasses * sel::kHistWords / 4; i += kThreads)
        reinterpret_cast<u32x4_t *>(sm.hist)[i] = u32x4_t{0u, 0u, 0u, 0u};
    uint32_t key[KMAX];
    src.fill(key, tid, kThreads, nb);
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
    for (int p = 0; p < sel::kTopkPasses && lo < hi; ++p) {
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
    __syncthreads();  // the histograms and red are reused by the caller
    return lo;  // a bin kept whole: exactly kb keys are >= lo; else lo = hi = the kb-th key
}

template <typename Src>
__device__ uint32_t kth_key(const Src &src, int nb, int kb, sel::TopkSmem &sm) {
    if (nb <= 4 * kThreads) return kth_key_wg4<4>(src, nb, kb, sm);
    if (nb <= 8 * kThreads) return kth_key_wg4<8>(src, nb, kb, sm);
    if (nb <= 16 * kThreads) return kth_key_wg4<16>(src, nb, kb, sm);
    return kth_key_wg4<32>(src, nb, kb, sm);
}

// Block ids j < nb with score_key(hi[j]) >= tau, in ascending order, into
// map[0 .. m) when m <= kCandCap; returns m (workgroup-uniform).
template <int KMAX>
__device__ int compact_candidates(const float *hi, int nb, uint32_t tau, int32_t *map,
                                  uint32_t *count, int *total) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    float hv[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) hv[i] = load_relaxed(hi + min(i * kThreads + tid, nb - 1));
    uint32_t flags = 0u;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const bool f = i * kThreads + tid < nb && score_key(hv[i]) >= tau;
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
    if (m <= kCandCap) {
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
    __syncthreads();
    return m;
}

__device__ int candidates(const float *hi, int nb, uint32_t tau, int32_t *map, uint32_t *count,
                          int *total) {
    if (nb <= 4 * kThreads) return compact_candidates<4>(hi, nb, tau, map, count, total);
    if (nb <= 8 * kThreads) return compact_candidates<8>(hi, nb, tau, map, count, total);
    if (nb <= 16 * kThreads) return compact_candidates<16>(hi, nb, tau, map, count, total);
    return compact_candidates<32>(hi, nb, tau, map, count, total);
}

// Interval ends of the sketch scores of blocks [j0, j0 + n) of unit (b, g):
// LPR lanes per row (16 codes each), KU rows per lane group in each of two
// stages in flight.  qs: the scaled mean query in sm.qs; q128 = 128 * sum(qs),
// qn1 = sum |qs|.
template <int D, int KU>
__device__ __forceinline__ void scan_sketch(const sel::SelectArgs &a, const SketchArgs &s, int b,
                                            int g, int j0, int n, const float *qs, float q128,
                                            float qn1) {
    constexpr int LPR = D / 16;          // lanes per row
    constexpr int RPW = kWave / LPR;     // rows per wave per load
    constexpr int ROWS = kWaves * RPW * KU;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int part = lane % LPR, rsub = lane / LPR;
    const size_t urow = ((size_t)b * a.Hkv + g) * a.max_blocks;
    float qf[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) qf[e] = qs[16 * part + e];
    const float ebase = kBoundFactor * qn1;
    struct Stage {
        u32x4_t c[KU];
        uint32_t h0[KU], h1[KU];
        int32_t pg[KU];
    };
    auto issue = [&](Stage &st, int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = min(base + u * kWaves * RPW + wave * RPW + rsub, n - 1);
            const size_t i = urow + j0 + row;
            st.c[u] = *reinterpret_cast<const u32x4_t *>(s.codes + i * D + 16 * part);
            const uint32_t *hp = reinterpret_cast<const uint32_t *>(s.hdr + i);
            st.h0[u] = hp[0];
            st.h1[u] = hp[1];
            st.pg[u] = a.bt[(size_t)b * a.max_blocks + j0 + row];
        }
    };
    auto reduce = [&](const Stage &st, int base) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int row = base + u * kWaves * RPW + wave * RPW + rsub;
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
            const int page = st.pg[u];
            const float scale = __uint_as_float(st.h1[u]);
            const bool valid = page >= 0 && page < a.num_pages && (int)st.h0[u] == page + 1;
            const float sa = scale * (t - q128);
            const float e = scale * ebase;
            if (part == 0 && row < n) {
                store_relaxed(s.lo + urow + j0 + row, valid ? sa - e : -INFINITY);
                store_relaxed(s.hi + urow + j0 + row, valid ? sa + e : INFINITY);
            }
        }
    };
    if (n > 0) {
        Stage sa_, sb_;
        issue(sa_, 0);
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

// One workgroup per (unit, chunk of blocks): sketch bounds of the chunk; the
// workgroup that completes the unit selects (threshold, candidates, exact
// scores of the candidates, top-k).
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 4) void select_sketch_kernel(sel::SelectArgs a,
                                                                    SketchArgs s) {
    __shared__ float qraw[kMaxGroup * D];
    __shared__ float qs[D];
    __shared__ int pages[kMaxChunk];
    __shared__ float sc_lds[kMaxChunk];
    __shared__ int is_last;
    __shared__ uint32_t hist[sel::kTopkPasses * sel::kHistWords], cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ int32_t cmap[kCandCap];
    __shared__ uint32_t ccount[32 * kWaves];
    __shared__ int ctotal;
    __shared__ float qsum_s[2];
    extern __shared__ uint32_t keys[];  // 512 words: top-k bitmaps beyond 2048 blocks
    sel::ScoreSmem sm{qraw, qs, pages, sc_lds, &is_last};
    sel::TopkSmem tk{hist, cand, red, scan_red, keys};
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int unit = blockIdx.x / a.nchunk_max, c = blockIdx.x % a.nchunk_max;
    const int b = unit / a.Hkv, g = unit % a.Hkv;
    int32_t *out = a.indices + (size_t)unit * a.top_k;
    const int j0 = c * a.chunk;

    // setup in one round trip: the group's queries and the length
    sel::load_setup<T, D, kMaxChunk>(a, b, g, j0, 0, sm);
    const int L = a.seq_lens[b];
    __syncthreads();
    if (L < 1 || L > a.max_blocks * kPage) {
        if (c == 0) {
            for (int i = tid; i < a.top_k; i += kThreads) store_relaxed_i32(out + i, -1);
            if (tid == 0) flag_error(a.err, kErrSeqLen);
        }
        return;
    }
    const int nb = (L + kPage - 1) / kPage;
    const int nchunks = (nb + a.chunk - 1) / a.chunk;
    if (c >= nchunks) return;
    const int n = min(nb, j0 + a.chunk) - j0;
    sel::mean_query<D>(a, sm);
    __syncthreads();
    if (wave == 0) {  // sum(qs) and sum|qs|
        float s0 = 0.f, s1 = 0.f;
        for (int d = lane; d < D; d += kWave) {
            s0 += qs[d];
            s1 += fabsf(qs[d]);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            s0 += __shfl_xor(s0, off);
            s1 += __shfl_xor(s1, off);
        }
        if (lane == 0) {
            qsum_s[0] = 128.f * s0;
            qsum_s[1] = s1;
        }
    }
    __syncthreads();
    scan_sketch<D, 4>(a, s, b, g, j0, n, qs, qsum_s[0], qsum_s[1]);
    if (!arrive_last(&a.counters[(size_t)unit * kStateStride], (uint32_t)nchunks, &is_last))
        return;

    // ---- the unit's selection
    const size_t urow = (size_t)unit * a.max_blocks;
    const int kb = min(a.top_k, nb);
    if (kb == nb) {  // every block is kept
        for (int i = tid; i < a.top_k; i += kThreads) store_relaxed_i32(out + i, i < nb ? i : -1);
        return;
    }
    const uint32_t tau = kth_key(sel::PlainScores{s.lo + urow}, nb, kb, tk);
    int m = candidates(s.hi + urow, nb, tau, cmap, ccount, &ctotal);
    const bool mapped = m <= kCandCap;
    if (!mapped) m = nb;  // every block is scored
    // exact scores of the candidates, in runs, with the select kernel's scan
    sel::SelectArgs ax = a;
    ax.scores = s.exact;
    for (int s0 = 0; s0 < m; s0 += kMaxChunk) {
        const int nr = min(kMaxChunk, m - s0);
        for (int t = tid; t < nr; t += kThreads) {
            const int j = mapped ? cmap[s0 + t] : s0 + t;
            pages[t] = a.bt[(size_t)b * a.max_blocks + j];
        }
        __syncthreads();
        sel::check_pages(a, sm, nr);
        __syncthreads();
        sel::scan_rows<T, D, 4, false>(ax, b, g, s0, nr, L, -1, sm, nullptr);
        __syncthreads();  // pages and sc_lds are reused by the next run
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the exact scores are stored
    __syncthreads();
    sel::TopkOut o{out};
    o.map = mapped ? cmap : nullptr;
    sel::select_topk(sel::PlainScores{s.exact + urow}, m, a.top_k, o, tk);
}

}  // namespace

size_t sketch_rows_offset(const Dims &d) {
    return ((size_t)d.B * d.Hkv * d.max_blocks * sizeof(SketchHdr) + 255) & ~(size_t)255;
}

size_t sketch_bytes(const Dims &d) {
    return sketch_rows_offset(d) + (size_t)d.B * d.Hkv * d.max_blocks * d.D;
}

hipError_t launch_sketch_update(const Dims &d, const float *centroids, const int32_t *block_table,
                                const int32_t *seq_lens, const int32_t *first_pos, void *sketch,
                                uint32_t *err, hipStream_t stream) {
    SketchHdr *hdr = static_cast<SketchHdr *>(sketch);
    uint8_t *codes = static_cast<uint8_t *>(sketch) + sketch_rows_offset(d);
    // decode (first_pos): one workgroup per unit over its touched blocks; a
    // full build: 256-block chunks
    const int per = first_pos ? d.max_blocks : 256;
    const int nch = (d.max_blocks + per - 1) / per;
    const size_t grid = (size_t)d.B * d.Hkv * nch;
    if (d.D == 128)
        hipLaunchKernelGGL(sketch_update_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, centroids, block_table, seq_lens, first_pos, d.Hkv,
                           d.max_blocks, d.num_pages, per, nch, hdr, codes, err);
    else
        hipLaunchKernelGGL(sketch_update_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, centroids, block_table, seq_lens, first_pos, d.Hkv,
                           d.max_blocks, d.num_pages, per, nch, hdr, codes, err);
    return hipGetLastError();
}

namespace {
template <typename T, int D>
hipError_t launch_sel(const Dims &d, sel::SelectArgs a, SketchArgs s, hipStream_t stream) {
    int cus = 0;
    hipError_t e = hipGetDevice(&cus);
    if (e != hipSuccess) return e;
    int dev = cus;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // chunks: as for btk_select, the smallest multiple of 64 blocks (from 256)
    // whose chunks all fit in one round of resident workgroups (four per CU)
    const size_t units = (size_t)d.B * d.Hkv, slots = (size_t)4 * (cus > 0 ? cus : 1);
    int chunk = 256;
    while (chunk < 8192 && units * (size_t)((d.max_blocks + chunk - 1) / chunk) > slots)
        chunk += 64;
    a.chunk = chunk;
    a.nchunk_max = (d.max_blocks + chunk - 1) / chunk;
    const size_t grid = units * a.nchunk_max;
    const size_t lds = d.max_blocks > 32 * kWave ? sizeof(uint32_t) * 512 : 0;
    hipLaunchKernelGGL((select_sketch_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), lds,
                       stream, a, s);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_select_sketch(const Dims &d, const void *q, const float *centroids,
                                const void *sketch, const int32_t *block_table,
                                const int32_t *seq_lens, int top_k, int32_t *indices,
                                float *lo, float *hi, float *exact, uint32_t *counters,
                                uint32_t *err, hipStream_t stream) {
    sel::SelectArgs a{q, centroids, block_table, seq_lens, indices, exact, counters, err,
                      d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, 0, 0,
                      d.sm_scale, nullptr, nullptr, nullptr};
    SketchArgs s{static_cast<const SketchHdr *>(sketch),
                 static_cast<const uint8_t *>(sketch) + sketch_rows_offset(d), lo, hi, exact};
    if (d.dtype == 0)
        return d.D == 128 ? launch_sel<uint16_t, 128>(d, a, s, stream)
                          : launch_sel<uint16_t, 64>(d, a, s, stream);
    return d.D == 128 ? launch_sel<float, 128>(d, a, s, stream)
                      : launch_sel<float, 64>(d, a, s, stream);
}

}  // namespace btk
