// Block sketches and the selection that uses them (S2 + S3 with the same
// result as btk_select).  (Pith review of "Kinetics: Rethinking Test-Time
// Scaling Laws", "What carries the argument": blocks are scored by their
// averaged keys and the k best are kept.  The sketch changes which centroid
// rows are read, not which blocks are selected.)  The row layout and the proof
// that the selection is unchanged are in sketch_dev.h.
#include "sketch_dev.h"

namespace btk {
namespace {

using sel::kThreads;
using sel::kWaves;
using sel::kMaxChunk;

using skt::SketchArgs;
using skt::SketchHdr;
constexpr int kCandCap = 2048;  // candidates whose block ids fit the LDS map

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
        skt::encode_row<D>(x, page, row, hdr, codes, lane);
    }
}

// ---- the selection ---------------------------------------------------------

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
    // read as 16-byte vectors (histogram bins, candidate keys): 16-byte aligned
    __shared__ __align__(16) uint32_t hist[sel::kTopkPasses * sel::kHistWords];
    __shared__ __align__(16) uint32_t cand[4 * kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    __shared__ int32_t cmap[kCandCap];
    __shared__ uint32_t ccount[32 * kWaves];
    __shared__ int ctotal;
    __shared__ float qsum_s[2];
    extern __shared__ uint32_t keys[];  // 512 words: top-k bitmaps beyond 2048 blocks
    sel::ScoreSmem sm{qraw, qs, pages, sc_lds, &is_last};
    sel::TopkSmem tk{hist, cand, red, scan_red, keys};
    const int tid = threadIdx.x;
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
    skt::query_sums<D>(qs, qsum_s);
    __syncthreads();
    // in runs of up to kMaxChunk blocks staged in LDS (sc_lds, and pages as floats)
    float *lo_lds = sc_lds, *hi_lds = reinterpret_cast<float *>(pages);
    for (int s0 = j0; s0 < j0 + n; s0 += kMaxChunk) {
        const int nr = min(kMaxChunk, j0 + n - s0);
        skt::scan_sketch<D, 1>(a, s, b, g, s0, nr, [&] { return make_int2(nr, nb); }, qs, qsum_s,
                               lo_lds, hi_lds, [] {});
        __syncthreads();
        skt::store_intervals(s, (size_t)unit * a.max_blocks, s0, nr, lo_lds, hi_lds);
        __syncthreads();  // the staging areas are reused
    }
    if (!arrive_last(&a.counters[(size_t)unit * kStateStride], (uint32_t)nchunks, &is_last))
        return;

    // ---- the unit's selection
    const size_t urow = (size_t)unit * a.max_blocks;
    const int kb = min(a.top_k, nb);
    if (kb == nb) {  // every block is kept
        for (int i = tid; i < a.top_k; i += kThreads) store_relaxed_i32(out + i, i < nb ? i : -1);
        return;
    }
    int m = skt::threshold_candidates(s.lo + urow, s.hi + urow, nb, kb, cmap, kCandCap, tk, ccount,
                                      &ctotal);
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
    o.map = cmap;
    o.mapped = mapped;
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
    // the selection only reads the sketch
    SketchHdr *hdr = static_cast<SketchHdr *>(const_cast<void *>(sketch));
    SketchArgs s{hdr, reinterpret_cast<uint8_t *>(hdr) + sketch_rows_offset(d), lo, hi, exact};
    if (d.dtype == 0)
        return d.D == 128 ? launch_sel<uint16_t, 128>(d, a, s, stream)
                          : launch_sel<uint16_t, 64>(d, a, s, stream);
    return d.D == 128 ? launch_sel<float, 128>(d, a, s, stream)
                      : launch_sel<float, 64>(d, a, s, stream);
}

}  // namespace btk
