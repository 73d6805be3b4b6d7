// S1: block centroid = mean of a page's valid keys, fp32 accumulation.
// (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What carries
// the argument": blocks are summarised by their averaged key vectors.)
//
// One wave per (page, KV head) block.  A key row of D elements is read as 16-byte
// vectors: LPR lanes cover one token row, TPI rows are read per instruction,
// so one wave instruction moves a contiguous 1 KiB of the token-major page.
// Partial sums over token rows are folded with cross-lane xor shuffles.
#include "btk_internal.h"

namespace btk {
namespace {

constexpr int kWavesPerWg = 4;

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
    static constexpr int n = 8;
    __device__ static void add(const void *p, float (&acc)[8]) {
        uint4 w = *reinterpret_cast<const uint4 *>(p);
        uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16_bits_to_f32(x[i] & 0xffffu);
            acc[2 * i + 1] += bf16_bits_to_f32(x[i] >> 16);
        }
    }
};
template <>
struct Vec16<float> {
    static constexpr int n = 4;
    __device__ static void add(const void *p, float (&acc)[4]) {
        float4 w = *reinterpret_cast<const float4 *>(p);
        acc[0] += w.x;
        acc[1] += w.y;
        acc[2] += w.z;
        acc[3] += w.w;
    }
};

// grid: x = block chunk (rebuild) or 1 (touched mode), y = KV head, z = sequence
template <typename T, int D>
__global__ __launch_bounds__(kWave * kWavesPerWg) void centroid_kernel(
    const T *__restrict__ k_cache, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ first_pos,
    float *__restrict__ centroids, int Hkv, int num_pages, int max_blocks, int blocks_per_wg) {
    constexpr int VEC = Vec16<T>::n;
    constexpr int LPR = D / VEC;       // lanes per token row
    constexpr int TPI = kWave / LPR;   // token rows per wave instruction
    static_assert(kWave % LPR == 0 && kPage % TPI == 0, "layout");

    const int b = blockIdx.z, g = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int L = seq_lens[b];
    if (L < 1 || L > max_blocks * kPage) return;
    const int nb = (L + kPage - 1) / kPage;
    int j0, j1;
    if (first_pos) {
        const int fp = first_pos[b];
        if (fp < 0 || fp >= L) return;
        j0 = fp / kPage;
        j1 = nb;
    } else {
        j0 = blockIdx.x * blocks_per_wg;
        j1 = min(nb, j0 + blocks_per_wg);
    }
    const int col = lane % LPR, row = lane / LPR;
    for (int j = j0 + wave; j < j1; j += kWavesPerWg) {
        const int page = block_table[(size_t)b * max_blocks + j];
        if (page < 0 || page >= num_pages) continue;
        const int v = min(kPage, L - j * kPage);
        const T *base = k_cache + ((size_t)page * Hkv + g) * kPage * D;
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
        for (int t0 = 0; t0 < kPage; t0 += TPI) {
            const int t = t0 + row;
            if (t < v) Vec16<T>::add(base + (size_t)t * D + col * VEC, acc);
        }
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
        }
        if (row == 0) {
            float *dst = centroids + ((size_t)page * Hkv + g) * D + col * VEC;
            const float vf = (float)v;
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                float4 o = make_float4(acc[e] / vf, acc[e + 1] / vf, acc[e + 2] / vf,
                                       acc[e + 3] / vf);
                *reinterpret_cast<float4 *>(dst + e) = o;
            }
        }
    }
}

template <typename T, int D>
hipError_t launch(const Dims &d, const void *k_cache, const int32_t *bt, const int32_t *sl,
                  const int32_t *fp, float *cent, hipStream_t stream) {
    const int per_wg = 4 * kWavesPerWg;  // rebuild mode: 16 blocks per workgroup
    dim3 grid(fp ? 1 : (d.max_blocks + per_wg - 1) / per_wg, d.Hkv, d.B);
    hipLaunchKernelGGL((centroid_kernel<T, D>), grid, dim3(kWave * kWavesPerWg), 0, stream,
                       static_cast<const T *>(k_cache), bt, sl, fp, cent, d.Hkv, d.num_pages,
                       d.max_blocks, per_wg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_centroid_update(const Dims &d, const void *k_cache, const int32_t *block_table,
                                  const int32_t *seq_lens, const int32_t *first_pos,
                                  float *centroids, hipStream_t stream) {
    if (d.dtype == 0) {
        return d.D == 128 ? launch<uint16_t, 128>(d, k_cache, block_table, seq_lens, first_pos,
                                                  centroids, stream)
                          : launch<uint16_t, 64>(d, k_cache, block_table, seq_lens, first_pos,
                                                 centroids, stream);
    }
    return d.D == 128
               ? launch<float, 128>(d, k_cache, block_table, seq_lens, first_pos, centroids, stream)
               : launch<float, 64>(d, k_cache, block_table, seq_lens, first_pos, centroids, stream);
}

}  // namespace btk
