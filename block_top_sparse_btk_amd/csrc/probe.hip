// Counter-calibration read: a kernel with a known number of algorithmic bytes
// and the request shape of the decode step's centroid scan (each lane loads 16
// bytes, half a wave covers one 512-byte row), so that hardware byte counters
// can be scaled against it.  It computes nothing of the method.
#include "btk_internal.h"

namespace btk {
namespace {

constexpr int kProbeRowWords = 32;  // 16-byte words per 512-byte row

__global__ void __launch_bounds__(256) row_read_probe_kernel(const u32x4_t *__restrict__ src,
                                                             int64_t src_rows,
                                                             const int32_t *__restrict__ row_ids,
                                                             int64_t rows,
                                                             uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int64_t waves = ((int64_t)gridDim.x * blockDim.x) / kWave;
    uint32_t acc = 0;
    for (int64_t i = 2 * wave + (lane >> 5); i < rows; i += 2 * waves) {
        const int64_t row = row_ids ? (int64_t)row_ids[i] : i;
        if (row < 0 || row >= src_rows) continue;
        const u32x4_t v = src[row * kProbeRowWords + (lane & (kProbeRowWords - 1))];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // a store that depends on every load and is almost never taken
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_row_read_probe(const void *src, int64_t src_rows, const int32_t *row_ids,
                                 int64_t rows, uint32_t *sink, hipStream_t stream) {
    const int64_t blocks = (rows + 7) / 8;  // 4 waves of 2 rows each
    const int grid = (int)(blocks < 8192 ? blocks : 8192);
    hipLaunchKernelGGL(row_read_probe_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4_t *>(src), src_rows, row_ids, rows, sink);
    return hipGetLastError();
}

}  // namespace btk
