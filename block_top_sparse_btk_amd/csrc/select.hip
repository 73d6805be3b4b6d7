// S2 + S3: group block scoring against fp32 centroids, then top-k per unit.
// (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What carries
// the argument": key blocks are scored by their averaged key vectors per query
// group and the top k blocks are retrieved.)
//
// Scoring is a bandwidth-bound GEMV: a unit (sequence b, KV head g) streams the
// n_b centroid rows (D fp32 = 512 B at D=128) named by its block table.  The
// unit's blocks are cut into chunks; one 256-thread workgroup scores one chunk.
// The r query heads of the group are folded into their mean on entry
// (linearity: the mean of the heads' logits equals the logit of the mean query),
// so each block costs one D-long dot product.  D/4 lanes hold one centroid row as
// 16-byte vectors and reduce it with xor shuffles; eight row loads per lane are
// kept in flight.
//
// Selection runs in the workgroup that finishes a unit's last chunk (a
// release/acquire counter per unit, reset by that workgroup), so it overlaps
// the scoring of later units and needs no extra launch.  It reads the unit's
// n_b scores back into LDS as order-preserving keys, binary-searches the k-th
// largest key with ballot counts, then takes every key above it plus the
// lowest-index keys equal to it, and writes the winners in ascending block
// order with two workgroup prefix scans.
#include "btk_internal.h"

namespace btk {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunk = 512;
constexpr int kUnroll = 8;

struct SelectArgs {
    const void *q;
    const float *cent;
    const int32_t *bt;
    const int32_t *seq_lens;
    int32_t *indices;
    float *scores;
    uint32_t *counters;
    uint32_t *err;
    int Hq, Hkv, num_pages, max_blocks, top_k, chunk, nchunk_max;
    float scale;
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

// keys: LDS scratch of at least nb words.  Counting passes read keys strided by
// thread (conflict-free); the final passes give thread t the contiguous range
// [t*R, t*R + R) so that thread order is block order.
__device__ void select_topk(const float *sc, int nb, int top_k, int32_t *out, uint32_t *keys) {
    __shared__ int red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    const int tid = threadIdx.x;
    const int kb = min(top_k, nb);
    if (kb == nb) {
        for (int i = tid; i < top_k; i += kThreads) out[i] = i < nb ? i : -1;
        return;
    }
    for (int j = tid; j < nb; j += kThreads) keys[j] = score_key(load_relaxed(sc + j));
    __syncthreads();
    const int R = (nb + kThreads - 1) / kThreads;  // keys per thread
    // largest T with #{key >= T} >= kb, i.e. the kb-th largest key (keys are >= 1)
    int parity = 0;
    uint32_t lo = 1u, hi = 0xffffffffu;
    while (lo < hi) {
        const uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
        int c = 0;
        for (int i = 0; i < R; ++i) {
            const int j = i * kThreads + tid;
            const uint32_t key = j < nb ? keys[j] : 0u;
            c += __popcll(__ballot(key >= mid));
        }
        c = wg_sum(c, red, parity);
        if (c >= kb) lo = mid;
        else hi = mid - 1;
    }
    const uint32_t T = lo;
    int gt = 0;
    if (T != 0xffffffffu) {
        int c = 0;
        for (int i = 0; i < R; ++i) {
            const int j = i * kThreads + tid;
            const uint32_t key = j < nb ? keys[j] : 0u;
            c += __popcll(__ballot(key > T));
        }
        gt = wg_sum(c, red, parity);
    }
    const int take_eq = kb - gt;  // keys equal to T to keep, lowest index first
    const int j0 = tid * R, j1 = min(nb, j0 + R);
    int my_eq = 0;
    for (int j = j0; j < j1; ++j) my_eq += keys[j] == T ? 1 : 0;
    const int eq_before = wg_exclusive_scan(my_eq, scan_red);
    int my_sel = 0;
    for (int j = j0, e = eq_before; j < j1; ++j) {
        const uint32_t key = keys[j];
        if (key > T || (key == T && e++ < take_eq)) ++my_sel;
    }
    int pos = wg_exclusive_scan(my_sel, scan_red);
    for (int j = j0, e = eq_before; j < j1; ++j) {
        const uint32_t key = keys[j];
        if ((key > T || (key == T && e++ < take_eq)) && pos < kb) out[pos++] = j;
    }
    for (int i = kb + tid; i < top_k; i += kThreads) out[i] = -1;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
    constexpr int LPR = D / 4;            // lanes per centroid row (16-byte vectors)
    constexpr int RPI = kWave / LPR;      // rows per wave instruction
    __shared__ float qs[D];
    __shared__ int pages[kMaxChunk];
    __shared__ int is_last;
    extern __shared__ uint32_t keys[];  // max_blocks words, used by the selecting workgroup

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int unit = blockIdx.x / a.nchunk_max, c = blockIdx.x % a.nchunk_max;
    const int b = unit / a.Hkv, g = unit % a.Hkv;
    const int r = a.Hq / a.Hkv;
    int32_t *out = a.indices + (size_t)unit * a.top_k;

    const int L = a.seq_lens[b];
    if (L < 1 || L > a.max_blocks * kPage) {
        if (c == 0) {
            for (int i = tid; i < a.top_k; i += kThreads) out[i] = -1;
            if (tid == 0) flag_error(a.err, kErrSeqLen);
        }
        return;
    }
    const int nb = (L + kPage - 1) / kPage;
    const int nchunks = (nb + a.chunk - 1) / a.chunk;
    if (c >= nchunks) return;
    const int j0 = c * a.chunk, n = min(nb, j0 + a.chunk) - j0;

    // group mean query, pre-scaled
    const T *qp = static_cast<const T *>(a.q) + ((size_t)b * a.Hq + (size_t)g * r) * D;
    for (int d = tid; d < D; d += kThreads) {
        float s = 0.f;
        for (int h = 0; h < r; ++h) s += load_q<T>(qp + (size_t)h * D + d);
        qs[d] = s * (a.scale / (float)r);
    }
    for (int i = tid; i < n; i += kThreads) {
        int p = a.bt[(size_t)b * a.max_blocks + j0 + i];
        if (p < 0 || p >= a.num_pages) {
            flag_error(a.err, kErrPage);
            p = -1;
        }
        pages[i] = p;
    }
    __syncthreads();

    const int col = lane % LPR, rsub = lane / LPR;
    const float4 qf = reinterpret_cast<const float4 *>(qs)[col];
    float *sc = a.scores + (size_t)unit * a.max_blocks;
    for (int base = wave * RPI; base < n; base += kWaves * RPI * kUnroll) {
        float4 cv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int row = base + u * kWaves * RPI + rsub;
            const int p = row < n ? pages[row] : -1;
            if (p >= 0)
                cv[u] = *reinterpret_cast<const float4 *>(
                    a.cent + ((size_t)p * a.Hkv + g) * D + col * 4);
            else
                cv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int row = base + u * kWaves * RPI + rsub;
            float s = qf.x * cv[u].x + qf.y * cv[u].y + qf.z * cv[u].z + qf.w * cv[u].w;
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
            if (col == 0 && row < n) store_relaxed(sc + j0 + row, pages[row] >= 0 ? s : -INFINITY);
        }
    }

    // the last workgroup of this unit selects
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&a.counters[unit], 1u);
        is_last = (prev == (uint32_t)(nchunks - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (tid == 0) a.counters[unit] = 0u;  // ready for the next call
    select_topk(sc, nb, a.top_k, out, keys);
}

template <typename T, int D>
hipError_t launch(const Dims &d, const SelectPlan &plan, SelectArgs a, hipStream_t stream) {
    const size_t grid = (size_t)d.B * d.Hkv * plan.nchunk_max;
    const size_t lds = sizeof(uint32_t) * (size_t)d.max_blocks;
    hipLaunchKernelGGL((select_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), lds, stream,
                       a);
    return hipGetLastError();
}

}  // namespace

SelectPlan plan_select(const Dims &d) {
    // Enough workgroups to cover 256 CUs several times over, with chunks large
    // enough that the per-workgroup setup (mean query, page list) stays small.
    const size_t rows = (size_t)d.B * d.Hkv * d.max_blocks;
    int chunk = 64;
    while (chunk < kMaxChunk && rows / (size_t)(chunk * 2) >= 2048) chunk *= 2;
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
                 d.sm_scale};
    if (d.dtype == 0)
        return d.D == 128 ? launch<uint16_t, 128>(d, plan, a, stream)
                          : launch<uint16_t, 64>(d, plan, a, stream);
    return d.D == 128 ? launch<float, 128>(d, plan, a, stream)
                      : launch<float, 64>(d, plan, a, stream);
}

}  // namespace btk
