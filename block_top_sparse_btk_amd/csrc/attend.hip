// S4 / S5 and the local-window baseline, stand-alone: one workgroup per (unit,
// split) (device code in attend_dev.h).
#include "attend_dev.h"

namespace btk {
using namespace att;
namespace {

// blocks per pipeline stage: one (fewer registers; the bf16 dense comparison on
// the Qwen3-8B-shaped layer took 488.7 instead of 501.6 us with one-block stages,
// while a third or fourth workgroup per CU gained nothing or spilled).
template <typename T, int MODE>
constexpr int stage_blocks() { return 1; }

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendArgs a) {
    extern __shared__ float smem[];
    __shared__ int is_last;
    attend_item<T, D, MODE, stage_blocks<T, MODE>()>(a, blockIdx.x / a.nsplit_max,
                                                  blockIdx.x % a.nsplit_max, smem, &is_last);
}

template <typename T, int D, int MODE>
hipError_t launch(const Dims &d, const AttendPlan &plan, AttendArgs a, hipStream_t stream) {
    const size_t grid = (size_t)d.B * d.Hkv * plan.nsplit_max;
    const size_t wave_merge = (size_t)kWaves * d.group() * D + 2 * kWaves * 16;
    const size_t split_merge = 2 * (size_t)plan.nsplit_max * d.group() + d.group();
    const size_t lds = sizeof(float) * (wave_merge > split_merge ? wave_merge : split_merge);
    hipLaunchKernelGGL((attend_kernel<T, D, MODE>), dim3((unsigned)grid), dim3(kThreads), lds,
                       stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dtype(const Dims &d, const AttendPlan &plan, int mode, AttendArgs a,
                        hipStream_t stream) {
    if (mode == kAll) return launch<T, D, kAll>(d, plan, a, stream);
    if (mode == kRecent) return launch<T, D, kRecent>(d, plan, a, stream);
    if (mode == kMasked) return launch<T, D, kMasked>(d, plan, a, stream);
    return launch<T, D, kSelected>(d, plan, a, stream);
}

}  // namespace

AttendPlan plan_attend(const Dims &d, int list_len_max, bool dense, int target) {
    // The split merge keeps nsplit * r maxima and normalisers in LDS: at most
    // kMaxSplitHeads of each.  A wave holds at most 64 list entries (one per lane).
    constexpr int kMaxSplitHeads = 2048;
    const size_t units = (size_t)d.B * d.Hkv;
    const int r = d.group();
    auto nsplit = [&](int bps) { return (list_len_max + bps - 1) / bps; };
    AttendPlan p;
    if (dense) {
        p.bps = 128;  // 32 blocks (256 KiB of bf16 K+V at D=128) per wave
    } else {
        // about `target` (256) workgroups (whole lists where that gives enough of them:
        // a split costs a round of partial stores and loads), each wave with
        // at least two blocks when the list allows it and at most 64, and the
        // list spread evenly over the four waves of a split
        const int want = (int)((target + units - 1) / units);
        int ns = want < list_len_max / 8 ? want : list_len_max / 8;
        if (ns < 1) ns = 1;
        if (ns < (list_len_max + 4 * kWave - 1) / (4 * kWave))
            ns = (list_len_max + 4 * kWave - 1) / (4 * kWave);
        p.bps = (list_len_max + ns - 1) / ns;
        p.bps = (p.bps + kWaves - 1) / kWaves * kWaves;
    }
    while (nsplit(p.bps) * r > kMaxSplitHeads && p.bps < 4 * kWave)
        p.bps = 2 * p.bps < 4 * kWave ? 2 * p.bps : 4 * kWave;
    p.nsplit_max = nsplit(p.bps);
    return p;
}

hipError_t launch_attend(const Dims &d, const AttendPlan &plan, int mode, const void *q,
                         const void *k_cache, const void *v_cache, const int32_t *block_table,
                         const int32_t *seq_lens, const int32_t *indices, int top_k, void *out,
                         float *lse, float *partials, uint32_t *counters, uint32_t *err,
                         hipStream_t stream, const uint32_t *counts) {
    AttendArgs a{q, k_cache, v_cache, block_table, seq_lens, indices, out, lse, partials,
                 counters, err, d.Hq, d.Hkv, d.num_pages, d.max_blocks, top_k, plan.bps,
                 plan.nsplit_max, d.sm_scale * 1.44269504088896340736f, counts};
    if (d.dtype == 0)
        return d.D == 128 ? launch_dtype<uint16_t, 128>(d, plan, mode, a, stream)
                          : launch_dtype<uint16_t, 64>(d, plan, mode, a, stream);
    return d.D == 128 ? launch_dtype<float, 128>(d, plan, mode, a, stream)
                      : launch_dtype<float, 64>(d, plan, mode, a, stream);
}

}  // namespace btk
