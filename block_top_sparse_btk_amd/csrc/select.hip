// S2 + S3 stand-alone: group block scoring and top-k selection in one launch
// (device code in select_dev.h).  Grid = units x chunks; the workgroup that
// finishes a unit's last chunk selects its top-k blocks.
#include "select_dev.h"

namespace btk {
using namespace sel;
namespace {

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
    __shared__ float qraw[kMaxGroup * D];
    __shared__ float qs[D];
    __shared__ int pages[kMaxChunk];
    __shared__ float sc_lds[kMaxChunk];
    __shared__ int is_last;
    __shared__ uint32_t hist[256 + kWave], cand[4 * kWave], above[kWave], equal[kWave];
    __shared__ uint32_t red[2 * kWaves];
    __shared__ int scan_red[kWaves];
    extern __shared__ uint32_t keys[];  // max_blocks words, long contexts only
    ScoreSmem sm{qraw, qs, pages, sc_lds, &is_last};
    TopkSmem tk{hist, cand, above, equal, red, scan_red, keys};
    const int unit = blockIdx.x / a.nchunk_max, c = blockIdx.x % a.nchunk_max;
    int nb = 0;
    if (!score_chunk<T, D, 4>(a, unit, c, sm, nullptr, nb)) return;
    // the selecting wave(s) take issue priority over scanning waves on the SIMD
    __builtin_amdgcn_s_setprio(3);
    select_topk(PlainScores{a.scores + (size_t)unit * a.max_blocks}, nb, a.top_k,
                TopkOut{a.indices + (size_t)unit * a.top_k, nullptr, 0u}, tk);
}

template <typename T, int D>
hipError_t launch(const Dims &d, const SelectPlan &plan, SelectArgs a, hipStream_t stream) {
    const size_t grid = (size_t)d.B * d.Hkv * plan.nchunk_max;
    // LDS key copy only for the workgroup-wide selection of long contexts
    const size_t lds = d.max_blocks > 32 * kWave ? sizeof(uint32_t) * (size_t)d.max_blocks : 0;
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
                 d.sm_scale, nullptr, nullptr, nullptr};
    if (d.dtype == 0)
        return d.D == 128 ? launch<uint16_t, 128>(d, plan, a, stream)
                          : launch<uint16_t, 64>(d, plan, a, stream);
    return d.D == 128 ? launch<float, 128>(d, plan, a, stream)
                      : launch<float, 64>(d, plan, a, stream);
}

}  // namespace btk
