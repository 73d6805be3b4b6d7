// S1: block centroid = mean of a page's valid keys, fp32 accumulation.
// (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What carries
// the argument": blocks are summarised by their averaged key vectors.)
//
// One wave per (page, KV head) block (block_centroid in centroid_dev.h).
#include "centroid_dev.h"

namespace btk {
namespace {

constexpr int kWavesPerWg = 4;

// grid: x = block chunk (rebuild) or 1 (touched mode), y = KV head, z = sequence
template <typename T, int D>
__global__ __launch_bounds__(kWave * kWavesPerWg) void centroid_kernel(
    const T *__restrict__ k_cache, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ first_pos,
    float *__restrict__ centroids, int Hkv, int num_pages, int max_blocks, int blocks_per_wg) {
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
    for (int j = j0 + wave; j < j1; j += kWavesPerWg) {
        const int page = block_table[(size_t)b * max_blocks + j];
        if (page < 0 || page >= num_pages) continue;
        const int v = min(kPage, L - j * kPage);
        block_centroid<T, D>(k_cache + ((size_t)page * Hkv + g) * kPage * D, v,
                             centroids + ((size_t)page * Hkv + g) * D, nullptr, lane);
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
