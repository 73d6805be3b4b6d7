// Token-level top-k baseline ("oracle top-k"): the group score of every valid
// token (a full key scan), the top_tokens best tokens of each unit, then exact
// attention over exactly those tokens.  (scime summary of "Kinetics: Rethinking
// Test-Time Scaling Law", "Experimental setup": oracle top-k attention is one of
// the baselines; "Limitations": the sparse results use it as their upper bound.)
// It is the block method with one-token blocks: a one-token block's mean key is
// the key itself, so the score of token t is scale * qbar . k_t and ties go to
// the lower position, as for blocks.
//
// token_score_kernel: grid = units x chunks of kChunkPages pages.  A workgroup
// scores its chunk's tokens (each load instruction of a wave reads 1 KiB of a
// key page contiguously, a group of lanes per key row, and a DPP sum over the
// group finishes the row's dot product) into the workspace, and adds its score
// range to the unit's.  Then token_select_kernel, one workgroup per unit,
// selects: a pass over score values (2048 equal bins across the unit's range,
// each bin's key extremes kept) and passes over key bits inside the threshold
// bin, each with a 2048-bin LDS histogram, find the K-th largest key T; one
// ordered pass over tiles of blocks (thread t takes block tile + t, so thread
// order is position order; workgroup prefix sums place the ties and the
// outputs) keeps every token above T plus the lowest-position tokens equal to
// T.  The result is written as packed entries (block | token mask << 16), one
// per block with a kept token, for the attention kernel's masked list mode, and
// as token positions when the caller asks for them.  (Selecting inside the
// scoring kernel, by the workgroup that completes a unit, made the scan itself
// more than twice as slow.)
#include "attend_dev.h"
#include "select_dev.h"

namespace btk {
namespace tok {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Pages scored per workgroup and pages per wave with loads in flight together.
// Measured on the Qwen3-8B-shaped layer (whole baseline call): 32 / 4 took
// 513 us, 64 / 2 482 us (fewer registers, more waves resident: 32 / 2 and 64 / 1
// were within 1 us of it), 128 / 2 486 us, 32 / 8 526 us.
constexpr int kChunkPages = 64;
constexpr int kUnroll = 2;
constexpr int kBins = 2048;  // radix bins per selection pass

struct TokArgs {
    const void *q, *k;
    const int32_t *bt, *seq_lens;
    float *scores;       // [units][max_blocks * 16]
    uint32_t *entries;   // [units][cap]: block | token mask << 16
    uint32_t *counts;    // [units]
    uint32_t *ranges;    // unit u: ranges[u * kStateStride] and the word after it, the
                         // max of ~key and the max of key over the unit's finite scores
                         // (0 0 = none; re-armed by the selector)
    int32_t *token_idx;  // [units][top_tokens] or NULL
    uint32_t *err;
    int Hq, Hkv, num_pages, max_blocks, top_tokens, cap, nchunk_max;
    float scale;
};

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
    return bf16_bits_to_f32(x);
}
template <>
__device__ __forceinline__ float to_f32<float>(float x) {
    return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (8, 16 or 32), in every lane of the group:
// quad xor 1 and 2, half-row mirror (8), row mirror (16), then across rows (32).
template <int N>
__device__ __forceinline__ float lanes_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    if (N >= 16) x += dpp_f<0x140>(x);
    if (N >= 32) x += __shfl_xor(x, 16);
    return x;
}

// Scores one chunk of a unit's tokens into the workspace and adds the chunk's
// finite score range to the unit's.
template <typename T, int D>
__device__ __forceinline__ void score_tokens(const TokArgs &a, int unit, int c, float *qraw,
                                             float *qs, int *pages) {
    constexpr int EV = 16 / (int)sizeof(T);  // elements per 16-byte load
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int b = unit / a.Hkv, g = unit % a.Hkv;
    const int r = a.Hq / a.Hkv;
    const int j0 = c * kChunkPages;
    const size_t max_tok = (size_t)a.max_blocks * kPage;

    // set-up in one round trip: queries, the chunk's slice of the block table,
    // the length.  The loads are unconditional (clamped addresses, surplus
    // results dropped): a conditional load compiles to a branch that waits for
    // it before the next is issued
    const T *qp = static_cast<const T *>(a.q) + ((size_t)b * a.Hq + (size_t)g * r) * D;
    constexpr int QN = (kMaxGroup * D + kThreads - 1) / kThreads;
    float qv[QN];
#pragma unroll
    for (int k = 0; k < QN; ++k) qv[k] = to_f32<T>(qp[min(k * kThreads + tid, r * D - 1)]);
    const int jn = min(kChunkPages, a.max_blocks - j0);
    static_assert(kChunkPages <= kThreads, "one page id per thread");
    const int pv = jn > 0 ? a.bt[(size_t)b * a.max_blocks + j0 + min(tid, jn - 1)] : -1;
#pragma unroll
    for (int k = 0; k < QN; ++k)
        if (k * kThreads + tid < r * D) qraw[k * kThreads + tid] = qv[k];
    if (tid < jn) pages[tid] = pv;
    const int L = a.seq_lens[b];
    __syncthreads();
    if (L < 1 || L > a.max_blocks * kPage) {
        if (c == 0 && tid == 0) flag_error(a.err, kErrSeqLen);
        return;
    }
    const int nb = (L + kPage - 1) / kPage;
    const int nchunks = (nb + kChunkPages - 1) / kChunkPages;
    if (c >= nchunks) return;
    const int n = min(nb, j0 + kChunkPages) - j0;
    for (int i = tid; i < n; i += kThreads) {
        const int p = pages[i];
        if (p < 0 || p >= a.num_pages) {
            flag_error(a.err, kErrPage);
            pages[i] = -1;
        }
    }
    if (tid < D) {
        float s = 0.f;
        for (int h = 0; h < r; ++h) s += qraw[h * D + tid];
        qs[tid] = s * (a.scale / (float)r);
    }
    __syncthreads();

    // Load instruction v of a page reads 1 KiB contiguous: lane l takes 16 bytes
    // of key row (token) v * RPI + l / LPR, LPR lanes per row; the row's dot
    // product ends in a DPP sum over those lanes.
    constexpr int LPR = D * (int)sizeof(T) / 16;  // lanes per key row (8, 16 or 32)
    constexpr int RPI = kWave / LPR;              // rows per load instruction
    constexpr int NI = kPage / RPI;               // load instructions per page
    const int col = lane % LPR, rsub = lane / LPR;
    float qf[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) qf[e] = qs[col * EV + e];
    float *sc = a.scores + (size_t)unit * max_tok;
    // kUnroll pages per wave step, loads unconditional (an invalid page reads
    // page 0 and a slot past the chunk its last page; neither result is kept)
    uint32_t kmin_c = 0u, kmax = 0u;  // max of ~key and of key over this lane's finite scores
    for (int i0 = wave; i0 < n; i0 += kWaves * kUnroll) {
        u32x4_t kv[kUnroll][NI];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = min(i0 + u * kWaves, n - 1);
            const int p = max(pages[i], 0);
            const u32x4_t *tile = reinterpret_cast<const u32x4_t *>(
                static_cast<const T *>(a.k) + ((size_t)p * a.Hkv + g) * kPage * D);
#pragma unroll
            for (int v = 0; v < NI; ++v) kv[u][v] = tile[v * kWave + lane];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = i0 + u * kWaves;
            const int j = j0 + i;
#pragma unroll
            for (int v = 0; v < NI; ++v) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < EV; ++e) s += qf[e] * vec16_elem<T>(kv[u][v], e);
                s = lanes_sum<LPR>(s);
                const int t = v * RPI + rsub;
                if (i < n && col == 0 && t < min(kPage, L - j * kPage)) {
                    store_relaxed(sc + (size_t)j * kPage + t, pages[i] >= 0 ? s : -INFINITY);
                    if (pages[i] >= 0 && s > -INFINITY && s < INFINITY) {
                        kmin_c = max(kmin_c, ~score_key(s));
                        kmax = max(kmax, score_key(s));
                    }
                }
            }
        }
    }
    // the chunk's score range joins the unit's (one atomic pair per wave)
    kmin_c = sel::wave_max_u32(kmin_c);
    kmax = sel::wave_max_u32(kmax);
    if (lane == 0 && kmax != 0u) {
        __hip_atomic_fetch_max(&a.ranges[(size_t)unit * kStateStride], kmin_c, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_max(&a.ranges[(size_t)unit * kStateStride + 1], kmax, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Exclusive prefix sum over the workgroup in thread order, and the total.
__device__ __forceinline__ int scan_total(int x, int *red, int &total) {
    const int before = sel::wg_exclusive_scan(x, red);
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += red[w];  // the waves' sums, set by the scan
    return before;
}

// The unit's top min(top_tokens, L) tokens, by the whole workgroup (see the
// file comment).  hist, bin_lo_c, bin_hi: kBins LDS words each; red, bcast:
// kWaves LDS words each.
// The scores were written by the scoring kernel (an earlier launch on the same
// stream), so plain loads see them; kKeys of them are in flight per thread.
__device__ __forceinline__ void select_tokens(const TokArgs &a, int unit, int L, uint32_t *hist,
                                              uint32_t *bin_lo_c, uint32_t *bin_hi, int *red,
                                              int *bcast) {
    constexpr int kKeys = 32;
    const int tid = threadIdx.x;
    const float *sc = a.scores + (size_t)unit * a.max_blocks * kPage;
    const int K = min(a.top_tokens, L);
    // f(score) for every score of the unit, kKeys loads per thread in flight
    auto for_scores = [&](auto &&f) {
        for (int base = 0; base < L; base += kThreads * kKeys) {
            float x[kKeys];
#pragma unroll
            for (int u = 0; u < kKeys; ++u) x[u] = sc[min(base + u * kThreads + tid, L - 1)];
#pragma unroll
            for (int u = 0; u < kKeys; ++u)
                if (base + u * kThreads + tid < L) f(x[u]);
        }
    };
    // the bin (from the top) holding rank `need`; need becomes the rank inside it
    auto locate = [&](int &need) {
        __syncthreads();
        uint32_t hb[kBins / kThreads];
        int sum = 0;
#pragma unroll
        for (int e = 0; e < kBins / kThreads; ++e) {
            hb[e] = hist[kBins - 1 - (kBins / kThreads) * tid - e];
            sum += (int)hb[e];
        }
        const int above = sel::wg_exclusive_scan(sum, red);
        if (above < need && above + sum >= need) {
            int acc = above;
#pragma unroll
            for (int e = 0; e < kBins / kThreads; ++e) {
                if (acc < need && acc + (int)hb[e] >= need) {
                    bcast[0] = kBins - 1 - (kBins / kThreads) * tid - e;
                    bcast[1] = need - acc;
                }
                acc += (int)hb[e];
            }
        }
        __syncthreads();
        const uint32_t b = (uint32_t)bcast[0];
        need = bcast[1];
        __syncthreads();  // bcast is rewritten by the next pass
        return b;
    };
    auto clear_hist = [&]() {
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
        __syncthreads();
    };
    // minimum and maximum over the workgroup (key order)
    auto wg_min_max = [&](uint32_t &lo, uint32_t &hi) {
        uint32_t mx = sel::wave_max_u32(hi), mn = ~sel::wave_max_u32(~lo);
        __syncthreads();
        if ((tid & (kWave - 1)) == 0) {
            red[tid / kWave] = (int)mx;
            bcast[tid / kWave] = (int)mn;
        }
        __syncthreads();
        lo = 0xffffffffu;
        hi = 0u;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            hi = max(hi, (uint32_t)red[w]);
            lo = min(lo, (uint32_t)bcast[w]);
        }
        __syncthreads();
    };
    int need = K;  // rank, from the top, of the K-th largest key among those in range

    // pass 1 over score values: 2048 equal bins between the finite minimum and
    // maximum (gathered while scoring), a non-decreasing function of the score,
    // so each bin holds a contiguous run of keys, whose extremes are kept per
    // bin (bins by key bits would crowd a few binades into a few bins)
    const uint32_t fl = ~a.ranges[(size_t)unit * kStateStride];
    const uint32_t fh = a.ranges[(size_t)unit * kStateStride + 1];
    __syncthreads();
    if (tid == 0) {  // re-armed for the next launch; every chunk has added its range
        __hip_atomic_store(&a.ranges[(size_t)unit * kStateStride], 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ranges[(size_t)unit * kStateStride + 1], 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t lo = 0u, hi = 0xffffffffu;  // the keys still in range
    if (fl < fh) {
        const float f_lo = __uint_as_float((fl & 0x80000000u) ? (fl & 0x7fffffffu) : ~fl);
        const float f_hi = __uint_as_float((fh & 0x80000000u) ? (fh & 0x7fffffffu) : ~fh);
        const float inv = (float)kBins / (f_hi - f_lo);
        if (inv > 0.f && inv < INFINITY) {
            for (int i = tid; i < kBins; i += kThreads) {
                hist[i] = 0u;
                bin_lo_c[i] = 0u;
                bin_hi[i] = 0u;
            }
            __syncthreads();
            for_scores([&](float x) {  // NaN goes to bin 0
                const uint32_t b = (uint32_t)fminf(fmaxf((x - f_lo) * inv, 0.f), (float)(kBins - 1));
                const uint32_t k = score_key(x);
                atomicAdd(&hist[b], 1u);
                atomicMax(&bin_lo_c[b], ~k);
                atomicMax(&bin_hi[b], k);
            });
            const uint32_t b = locate(need);
            lo = ~bin_lo_c[b];
            hi = bin_hi[b];
            __syncthreads();
        }
    }
    if (lo == 0u && hi == 0xffffffffu) {  // no usable value range: all keys
        uint32_t l = 0xffffffffu, h = 0u;
        for_scores([&](float x) {
            l = min(l, score_key(x));
            h = max(h, score_key(x));
        });
        wg_min_max(l, h);
        lo = l;
        hi = h;
    }
    // then passes over key bits inside [lo, hi], 11 bits each
    while (lo < hi) {
        const uint32_t span = hi - lo;
        const int shift = max(0, 21 - __builtin_clz(span));  // (span >> shift) < 2048
        clear_hist();
        for_scores([&](float x) {
            const uint32_t off = score_key(x) - lo;
            if (off <= span) atomicAdd(&hist[off >> shift], 1u);
        });
        const uint32_t b = locate(need);
        const uint32_t top = (b << shift) + ((1u << shift) - 1u);
        if (top < span) hi = lo + top;
        lo += b << shift;
    }
    const uint32_t prefix = lo;
    const uint32_t Tk = prefix;  // the K-th largest key
    const int take_eq = need;    // keys equal to Tk to keep, lowest positions first

    // Tiles of kThreads blocks, thread t taking block tile + t (thread order is
    // position order); running totals carry the tie count and output positions.
    const int nb = (L + kPage - 1) / kPage;
    uint32_t *ent = a.entries + (size_t)unit * a.cap;
    int32_t *tix = a.token_idx ? a.token_idx + (size_t)unit * a.top_tokens : nullptr;
    int carry_eq = 0, carry_sel = 0, carry_blk = 0;
    for (int jt = 0; jt < nb; jt += kThreads) {
        const int j = jt + tid;
        const int v = j < nb ? min(kPage, L - j * kPage) : 0;
        uint32_t k[kPage];
#pragma unroll
        for (int t = 0; t < kPage; ++t)
            k[t] = score_key(sc[(size_t)min(j, nb - 1) * kPage + min(t, max(v, 1) - 1)]);
        int eq = 0;
#pragma unroll
        for (int t = 0; t < kPage; ++t) eq += (t < v && k[t] == Tk) ? 1 : 0;
        int tot = 0;
        int e = carry_eq + scan_total(eq, red, tot);
        carry_eq += tot;
        uint32_t m = 0u;
#pragma unroll
        for (int t = 0; t < kPage; ++t) {
            if (t < v && (k[t] > Tk || (k[t] == Tk && e < take_eq))) m |= 1u << t;
            if (t < v && k[t] == Tk) ++e;
        }
        int pos = carry_sel + scan_total(__popc(m), red, tot);
        carry_sel += tot;
        const int bp = carry_blk + scan_total(m ? 1 : 0, red, tot);
        carry_blk += tot;
        if (m) ent[bp] = (uint32_t)j | (m << 16);
        if (tix)
            for (uint32_t mm = m; mm; mm &= mm - 1u) tix[pos++] = j * kPage + __builtin_ctz(mm);
    }
    if (tix)
        for (int i = K + tid; i < a.top_tokens; i += kThreads) tix[i] = -1;
    if (tid == 0) a.counts[unit] = (uint32_t)carry_blk;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void token_score_kernel(TokArgs a) {
    __shared__ float qraw[kMaxGroup * D];
    __shared__ float qs[D];
    __shared__ int pages[kChunkPages];
    score_tokens<T, D>(a, blockIdx.x / a.nchunk_max, blockIdx.x % a.nchunk_max, qraw, qs, pages);
}

// one workgroup per unit, after every unit has been scored
__global__ __launch_bounds__(kThreads) void token_select_kernel(TokArgs a) {
    __shared__ uint32_t hist[kBins], bin_lo_c[kBins], bin_hi[kBins];
    __shared__ int red[kWaves], bcast[kWaves];
    const int unit = blockIdx.x, b = unit / a.Hkv;
    const int L = a.seq_lens[b];
    if (L < 1 || L > a.max_blocks * kPage) {  // flagged by the scoring kernel
        if (threadIdx.x == 0) a.counts[unit] = 0u;
        if (a.token_idx)
            for (int i = threadIdx.x; i < a.top_tokens; i += kThreads)
                a.token_idx[(size_t)unit * a.top_tokens + i] = -1;
        return;
    }
    select_tokens(a, unit, L, hist, bin_lo_c, bin_hi, red, bcast);
}

template <typename T, int D>
hipError_t launch(const Dims &d, TokArgs a, hipStream_t stream) {
    const size_t units = (size_t)d.B * d.Hkv;
    hipLaunchKernelGGL((token_score_kernel<T, D>), dim3((unsigned)(units * a.nchunk_max)),
                       dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(token_select_kernel, dim3((unsigned)units), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tok

hipError_t launch_token_select(const Dims &d, const void *q, const void *k_cache,
                               const int32_t *block_table, const int32_t *seq_lens,
                               int top_tokens, int cap, float *scores, uint32_t *counters,
                               uint32_t *entries, uint32_t *counts, uint32_t *ranges,
                               int32_t *token_idx, uint32_t *err, hipStream_t stream) {
    (void)counters;
    tok::TokArgs a{q,       k_cache, block_table, seq_lens, scores,
                   entries, counts,  ranges,      token_idx, err,      d.Hq,   d.Hkv,
                   d.num_pages, d.max_blocks, top_tokens, cap,
                   (d.max_blocks + tok::kChunkPages - 1) / tok::kChunkPages, d.sm_scale};
    if (d.dtype == 0)
        return d.D == 128 ? tok::launch<uint16_t, 128>(d, a, stream)
                          : tok::launch<uint16_t, 64>(d, a, stream);
    return d.D == 128 ? tok::launch<float, 128>(d, a, stream) : tok::launch<float, 64>(d, a, stream);
}

}  // namespace btk
