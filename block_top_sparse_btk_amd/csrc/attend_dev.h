// Device code of S4 / S5 (attention of a query group over a list of KV
// blocks), shared by the stand-alone attention kernels and the single-launch
// decode step.
// S4 / S5: exact softmax attention of a query group over a list of KV blocks
// (the selected blocks, or every block for the dense comparison).
// (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws", "What carries
// the argument": attention runs over only the retrieved top-k blocks; the dense
// path is the paged decode attention it is compared with, Kinetics README
// (GitLite mirror), "Benchmark Block TopK Attention throughput".)
//
// Work unit: one (sequence, KV head) pair and a split of its block list; one
// 256-thread workgroup per split, its four waves take contiguous runs of the
// split.  A wave handles the r query heads of the group at once with MFMA
// tiles whose 16 rows cover the group (rows >= r are zero queries):
//   S^T[t][h] = K_tile (16 tokens x D) . Q^T        (16x16x32 bf16 / 16x16x4 f32)
// The 16x16 fp32 result leaves lane l holding tokens 4*(l/16)+e of head l%16,
// which is exactly the A-operand layout of the next product, so probabilities
// never leave registers:
//   O[h][d] += P (heads x 16 tokens) . V_tile (16 tokens x D)   (16x16x16 bf16)
// V pages are stored dim-major ([D][16] per page and head), so each lane's
// B operand (4 consecutive tokens of one dimension) is one 8-byte load and a
// wave instruction reads 512 contiguous bytes.  K pages are token-major and each
// lane reads 16 contiguous bytes per K instruction.
// Online softmax runs per group of G blocks in the base-2 domain with the
// scale folded in; the P fed to the bf16 product is rounded to bf16, while the
// normaliser and the log-sum-exp sum the unrounded weights.  Blocks are
// double-buffered: the loads of the next group are in flight while the current
// one is computed.
// Waves merge through LDS; splits merge through the workspace in the
// workgroup that finishes last (a counter per unit, see arrive_last).
#pragma once
#include <type_traits>

#include "btk_internal.h"

namespace btk {
namespace att {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kLn2 = 0.69314718055994530942f;

template <typename T, int D>
struct Mfma;

// bf16: QK with v_mfma_f32_16x16x32_bf16, PV with v_mfma_f32_16x16x16_bf16.
template <int D>
struct Mfma<uint16_t, D> {
    static constexpr int NK = D / 32;
    static constexpr int NV = D / 16;
    struct KFrag {
        bf16x8_t x[NK];
    };
    struct VFrag {
        short4_t x[NV];
    };
    using QFrag = KFrag;

    // lane l: token l%16, dims 32*i + 8*(l/16) .. +8
    __device__ static void load_k(KFrag &f, const uint16_t *tile, int lane) {
        const uint16_t *p = tile + (lane & 15) * D + 8 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < NK; ++i) f.x[i] = *reinterpret_cast<const bf16x8_t *>(p + 32 * i);
    }
    // lane l: head l%16 (zero when >= r), same dims as load_k
    __device__ static void load_q(QFrag &f, const uint16_t *qg, int r, int lane) {
        const int h = lane & 15;
        const uint16_t *p = qg + h * D + 8 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < NK; ++i)
            f.x[i] = h < r ? *reinterpret_cast<const bf16x8_t *>(p + 32 * i)
                           : __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
    __device__ static floatx4_t qk(const KFrag &k, const QFrag &q) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.x[i], q.x[i], acc, 0, 0, 0);
        return acc;
    }
    // lane l: dim 16*n + l%16, tokens 4*(l/16) .. +4 of the dim-major tile
    __device__ static void load_v(VFrag &f, const uint16_t *tile, int lane) {
        const uint16_t *p = tile + (lane & 15) * kPage + 4 * (lane >> 4);
#pragma unroll
        for (int n = 0; n < NV; ++n) f.x[n] = *reinterpret_cast<const short4_t *>(p + 16 * kPage * n);
    }
    // zero the values of tokens outside `mask` (bit t = token t of the page)
    __device__ static void mask_v(VFrag &f, uint32_t mask, int lane) {
        const int t0 = 4 * (lane >> 4);
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!((mask >> (t0 + e)) & 1u)) f.x[n][e] = 0;
    }
    __device__ static float round_p(float p) { return bf16_bits_to_f32(f32_to_bf16_bits(p)); }
    __device__ static void pv(floatx4_t (&o)[NV], const float (&p)[4], const VFrag &v) {
        short4_t a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (short)(__float_as_uint(p[e]) >> 16);  // p is bf16-exact
#pragma unroll
        for (int n = 0; n < NV; ++n)
            o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, v.x[n], o[n], 0, 0, 0);
    }
};

// fp32: both products with v_mfma_f32_16x16x4f32 (one k-slot per lane group).
template <int D>
struct Mfma<float, D> {
    static constexpr int NK = D / 4;
    static constexpr int NV = D / 16;
    struct KFrag {
        floatx4_t x[NK / 4];  // element i of the k-slots: x[i / 4][i % 4]
    };
    struct VFrag {
        floatx4_t x[NV];
    };
    using QFrag = KFrag;

    // lane l: token l%16, dims (l/16)*(D/4) + i
    __device__ static void load_k(KFrag &f, const float *tile, int lane) {
        const float *p = tile + (lane & 15) * D + (lane >> 4) * (D / 4);
#pragma unroll
        for (int i = 0; i < NK / 4; ++i) f.x[i] = *reinterpret_cast<const floatx4_t *>(p + 4 * i);
    }
    __device__ static void load_q(QFrag &f, const float *qg, int r, int lane) {
        const int h = lane & 15;
        const float *p = qg + h * D + (lane >> 4) * (D / 4);
#pragma unroll
        for (int i = 0; i < NK / 4; ++i)
            f.x[i] = h < r ? *reinterpret_cast<const floatx4_t *>(p + 4 * i)
                           : floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    __device__ static floatx4_t qk(const KFrag &k, const QFrag &q) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.x[i / 4][i % 4], q.x[i / 4][i % 4], acc,
                                                       0, 0, 0);
        return acc;
    }
    // lane l: dim 16*n + l%16, tokens 4*(l/16) .. +4
    __device__ static void load_v(VFrag &f, const float *tile, int lane) {
        const float *p = tile + (lane & 15) * kPage + 4 * (lane >> 4);
#pragma unroll
        for (int n = 0; n < NV; ++n) f.x[n] = *reinterpret_cast<const floatx4_t *>(p + 16 * kPage * n);
    }
    __device__ static void mask_v(VFrag &f, uint32_t mask, int lane) {
        const uint32_t m = mask >> (4 * (lane >> 4));
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!((m >> e) & 1u)) f.x[n][e] = 0.f;
    }
    __device__ static float round_p(float p) { return p; }
    // MFMA e contracts token 4*(l/16)+e of every lane group
    __device__ static void pv(floatx4_t (&o)[NV], const float (&p)[4], const VFrag &v) {
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[e], v.x[n][e], o[n], 0, 0, 0);
    }
};

struct AttendArgs {
    const void *q, *k, *v;
    const int32_t *bt, *seq_lens, *indices;
    void *out;
    float *lse, *partials;
    uint32_t *counters, *err;  // unit u's arrival counter at counters[u * kStateStride]
    int Hq, Hkv, num_pages, max_blocks, top_k, bps, nsplit_max;
    float scale_log2;
    // token-level baseline only (NULL otherwise): the number of packed entries
    // (block | token mask << 16) per unit in `indices`
    const uint32_t *counts;
};

// Tokens 0 .. v-1 of a page.
__device__ __forceinline__ uint32_t valid_mask(int v) {
    return v >= kPage ? 0xFFFFu : (1u << v) - 1u;
}

// K and V fragments of N blocks (one pipeline stage).
template <typename F, int N>
struct Stage {
    static constexpr int kN = N;
    typename F::KFrag k[N];
    typename F::VFrag v[N];
};

template <typename T>
__device__ __forceinline__ void store_out(T *p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float x) {
    *p = (uint16_t)f32_to_bf16_bits(x);
}
template <>
__device__ __forceinline__ void store_out<float>(float *p, float x) {
    *p = x;
}

// Which block list an item attends over: the unit's selection (S4), every block
// of the sequence (S5, the dense comparison), the most recent min(top_k, n_b)
// blocks (the local-window baseline, where top_k is the window in blocks), or
// counts[unit] packed entries (block | token mask << 16) of the token-level
// baseline, where top_k is the list capacity and only the masked tokens count.
enum ListMode : int { kSelected = 0, kAll = 1, kRecent = 2, kMasked = 3 };

// One (unit, split) item: attention of the unit's query group over its share of
// the block list, kG blocks per pipeline stage.  smem: the wave-merge /
// split-merge area (see launch sizing); is_last: one LDS word.  The decode
// step, which selects in the same workgroup, also passes what it already holds:
// lds_list, the split's share of the selection in LDS (entry i of the list at
// lds_list[i - split * bps]) instead of a.indices; L_known >= 0, the sequence
// length; lds_pages (or NULL), the sequence's block-table row in LDS.
// SPLITS = false: the caller guarantees one split per unit (nsplit_max = 1), and
// the split-merge code is left out of the instance.
template <typename T, int D, int MODE, int kG, bool SPLITS = true>
__device__ __forceinline__ void attend_item(const AttendArgs &a, int unit, int split, float *smem,
                                            int *is_last_p, const int32_t *lds_list = nullptr,
                                            int L_known = -1,
                                            const int32_t *lds_pages = nullptr) {
    using F = Mfma<T, D>;
    constexpr int NV = F::NV;
    int &is_last = *is_last_p;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int b = unit / a.Hkv, g = unit % a.Hkv;
    const int r = a.Hq / a.Hkv;
    constexpr bool LISTED = MODE == kSelected || MODE == kMasked;
    // a selection has top_k entries whatever the length, so its entries are
    // requested together with the length
    const int per_wave = a.bps / kWaves;
    int cnt = 0, w0 = 0;
    uint32_t entry = 0;
    if (LISTED) {
        const int i0 = split * a.bps, i1 = min(a.top_k, i0 + a.bps);
        w0 = i0 + wave * per_wave;
        cnt = max(0, min(i1, w0 + per_wave) - w0);
        if (lane < cnt)
            entry = (uint32_t)(lds_list ? lds_list[w0 - i0 + lane]
                                        : a.indices[(size_t)unit * a.top_k + w0 + lane]);
    }
    const int L = L_known >= 0 ? L_known : a.seq_lens[b];
    const int count = MODE == kMasked ? (int)a.counts[unit] : 0;
    if (L < 1 || L > a.max_blocks * kPage) {
        if (split == 0 && tid == 0) flag_error(a.err, kErrSeqLen);
        return;
    }
    const int nb = (L + kPage - 1) / kPage;
    const int len = MODE == kAll      ? nb
                    : MODE == kRecent ? min(a.top_k, nb)
                    : MODE == kMasked ? min(count, a.top_k)
                                      : a.top_k;
    const int nsplit = (len + a.bps - 1) / a.bps;
    if (split >= nsplit) return;
    if (MODE == kMasked) cnt = max(0, min(cnt, len - w0));
    if (!LISTED) {
        const int i0 = split * a.bps, i1 = min(len, i0 + a.bps);
        w0 = i0 + wave * per_wave;
        cnt = max(0, min(i1, w0 + per_wave) - w0);
    }

    // lane m < cnt holds page id and token mask (bit t: token t of the page is
    // attended) of this wave's m-th entry (page -1 and mask 0 for a skipped or
    // invalid entry)
    int my_page = -1;
    uint32_t my_mask = 0u;
    if (lane < cnt) {
        int j = MODE == kMasked ? (int)(entry & 0xFFFFu)
                : LISTED        ? (int32_t)(uint32_t)entry
                                : nb - len + w0 + lane;  // kAll: len = nb
        const uint32_t entry_mask = MODE == kMasked ? (uint32_t)(entry >> 16) & 0xFFFFu : 0xFFFFu;
        if (LISTED && j >= nb) {
            flag_error(a.err, kErrIndex);
            j = -1;
        }
        if (j >= 0) {
            const int p = lds_pages ? lds_pages[j] : a.bt[(size_t)b * a.max_blocks + j];
            if (p >= 0 && p < a.num_pages) {
                my_page = p;
                my_mask = valid_mask(min(kPage, L - j * kPage)) & entry_mask;
            } else {
                flag_error(a.err, kErrPage);
            }
        }
    }

    const T *qg = static_cast<const T *>(a.q) + ((size_t)b * a.Hq + (size_t)g * r) * D;
    typename F::QFrag qf;
    F::load_q(qf, qg, r, lane);
    const size_t page_stride = (size_t)a.Hkv * kPage * D;
    const T *kbase = static_cast<const T *>(a.k) + (size_t)g * kPage * D;
    const T *vbase = static_cast<const T *>(a.v) + (size_t)g * kPage * D;

    float m_run = -INFINITY, z_run = 0.f;
    floatx4_t o[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) o[n] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // Loads and their consumers are unconditional, so the compiler can keep
    // the next stage in flight (precise vmcnt) while the current one computes:
    // a slot past the wave's list re-reads its last entry (a cache hit) and an
    // invalid entry reads page 0; both are masked to zero weight below.
    const int safe_page = my_page >= 0 ? my_page : 0;
    auto issue = [&](auto &s, int m0) {
        constexpr int kN = std::remove_reference_t<decltype(s)>::kN;
#pragma unroll
        for (int u = 0; u < kN; ++u) {
            const int m = min(m0 + u, cnt - 1);
            const int page = __builtin_amdgcn_readlane(safe_page, m);
            F::load_k(s.k[u], kbase + page * page_stride, lane);
            F::load_v(s.v[u], vbase + page * page_stride, lane);
        }
    };
    auto compute = [&](auto &s, int m0) {
        constexpr int kN = std::remove_reference_t<decltype(s)>::kN;
        float sv[kN][4];
        uint32_t mk[kN];
        float gmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < kN; ++u) {
            const int m = min(m0 + u, cnt - 1);
            // token mask of this slot, 0 for a repeated or invalid entry (wave-uniform)
            mk[u] = m0 + u < cnt ? (uint32_t)__builtin_amdgcn_readlane((int)my_mask, m) : 0u;
            const floatx4_t acc = F::qk(s.k[u], qf);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * (lane >> 4) + e;
                sv[u][e] = ((mk[u] >> t) & 1u) ? acc[e] * a.scale_log2 : -INFINITY;
                gmax = fmaxf(gmax, sv[u][e]);
            }
        }
        gmax = fmaxf(gmax, __shfl_xor(gmax, 16));
        gmax = fmaxf(gmax, __shfl_xor(gmax, 32));
        const float m_new = fmaxf(m_run, gmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing valid yet: keep zeros
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 when m_run = -inf
        z_run *= alpha;
        // O rows are heads 4*(l/16)+e; alpha of head h lives in lane h
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ar = __shfl(alpha, 4 * (lane >> 4) + e);
#pragma unroll
            for (int n = 0; n < NV; ++n) o[n][e] *= ar;
        }
        m_run = m_new;
#pragma unroll
        for (int u = 0; u < kN; ++u) {
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pe = __builtin_amdgcn_exp2f(sv[u][e] - m_use);  // 0 for masked tokens
                z_run += pe;  // the normaliser (and lse) use the unrounded weights
                p[e] = F::round_p(pe);
            }
            if (mk[u] != 0xFFFFu) F::mask_v(s.v[u], mk[u], lane);  // no 0 * garbage in P.V
            F::pv(o, p, s.v[u]);
        }
    };

    if (cnt > 0) {
        Stage<F, kG> sa, sb;
        issue(sa, 0);
        for (int m0 = 0;;) {
            issue(sb, m0 + kG);
            compute(sa, m0);
            m0 += kG;
            if (m0 >= cnt) break;
            issue(sa, m0 + kG);
            compute(sb, m0);
            m0 += kG;
            if (m0 >= cnt) break;
        }
    }

    // ---- merge the four waves through LDS
    float *so = smem;                          // [kWaves][r][D]
    float *sm = smem + kWaves * r * D;         // [kWaves][16]
    float *sz = sm + kWaves * 16;              // [kWaves][16]
    float z = z_run;
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    if (lane < 16) {
        sm[wave * 16 + lane] = m_run;
        sz[wave * 16 + lane] = z;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = 4 * (lane >> 4) + e;
        if (h < r) {
#pragma unroll
            for (int n = 0; n < NV; ++n) so[(wave * r + h) * D + 16 * n + (lane & 15)] = o[n][e];
        }
    }
    __syncthreads();

    const int row = 2 * r + r * D;  // floats per partial: o[r][D], m[r], z[r]
    float *part = a.partials + ((size_t)unit * a.nsplit_max + split) * row;
    T *outp = static_cast<T *>(a.out) + ((size_t)b * a.Hq + (size_t)g * r) * D;
    for (int idx = tid; idx < r * D; idx += kThreads) {
        const int h = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * 16 + h]);
        float acc = 0.f, Z = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = sm[w * 16 + h];
                if (mw > -INFINITY) {
                    const float s = __builtin_amdgcn_exp2f(mw - M);
                    acc += s * so[(w * r + h) * D + d];
                    Z += s * sz[w * 16 + h];
                }
            }
        }
        if (!SPLITS || nsplit == 1) {
            store_out<T>(outp + (size_t)h * D + d, acc / Z);
            if (d == 0 && a.lse) a.lse[(size_t)b * a.Hq + (size_t)g * r + h] = M * kLn2 + logf(Z);
        } else {
            store_relaxed(part + idx, acc);
            if (d == 0) {
                store_relaxed(part + r * D + h, M);
                store_relaxed(part + r * D + r + h, Z);
            }
        }
    }
    if (!SPLITS || nsplit == 1) return;

    // ---- the last split of this unit merges all splits
    if (!arrive_last(&a.counters[(size_t)unit * kStateStride], (uint32_t)nsplit, &is_last)) return;
    // split weights: every (split, head) max and normaliser fetched at once into
    // LDS (reusing the wave-merge area), then w[s][h] = exp2(m_s - M_h)
    float *wm = smem;                  // [nsplit][r] split maxima, then weights
    float *wz = smem + nsplit * r;     // [nsplit][r] split normalisers
    float *hz = wz + nsplit * r;       // [r] merged normaliser
    __syncthreads();                   // the wave-merge area is free again
    const float *parts = a.partials + (size_t)unit * a.nsplit_max * row;
    // With few splits the split outputs are requested together with the maxima
    // and normalisers (one round trip instead of two): at most 4 splits of at
    // most 4 values per thread, held in registers until the weights are known
    // (the four-split steps of 64 units took 2.5-2.8 us less; allowing 8 splits
    // gained less, from the registers it holds).
    constexpr int kFastSplits = 4, kFastPer = 4;
    const bool fast = nsplit <= kFastSplits && r * D <= kFastPer * kThreads;
    float ov[kFastPer][kFastSplits];
    if (fast) {
#pragma unroll
        for (int i = 0; i < kFastPer; ++i) {
            const int idx = tid + i * kThreads;
            const float *src = parts + min(idx, r * D - 1);  // per-lane address, advanced by row
#pragma unroll
            for (int sp = 0; sp < kFastSplits; ++sp) {
                ov[i][sp] = sp < nsplit ? load_relaxed(src) : 0.f;
                src += row;
            }
        }
    }
    for (int i = tid; i < nsplit * r; i += kThreads) {
        const int sp = i / r, h = i % r;
        wm[i] = load_relaxed(parts + (size_t)sp * row + r * D + h);
        wz[i] = load_relaxed(parts + (size_t)sp * row + r * D + r + h);
    }
    __syncthreads();
    if (tid < r) {
        float M = -INFINITY;
        for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, wm[sp * r + tid]);
        float Z = 0.f;
        for (int sp = 0; sp < nsplit; ++sp) {
            const float ms = wm[sp * r + tid];
            const float w = ms > -INFINITY ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
            wm[sp * r + tid] = w;
            Z += w * wz[sp * r + tid];
        }
        hz[tid] = Z;
        if (a.lse) a.lse[(size_t)b * a.Hq + (size_t)g * r + tid] = M * kLn2 + logf(Z);
    }
    __syncthreads();
    if (fast) {  // the same sums, in the same order, from registers
#pragma unroll
        for (int i = 0; i < kFastPer; ++i) {
            const int idx = tid + i * kThreads;
            if (idx < r * D) {
                const int h = idx / D;
                float acc = 0.f;
#pragma unroll
                for (int sp = 0; sp < kFastSplits; ++sp)
                    if (sp < nsplit) acc += wm[sp * r + h] * ov[i][sp];
                store_out<T>(outp + idx, acc / hz[h]);
            }
        }
        return;
    }
    // weighted sum of the split outputs: loads of eight splits in flight per thread
    for (int idx = tid; idx < r * D; idx += kThreads) {
        const int h = idx / D;
        float acc = 0.f;
        int sp = 0;
        for (; sp + 8 <= nsplit; sp += 8) {
            float o8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) o8[u] = load_relaxed(parts + (size_t)(sp + u) * row + idx);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += wm[(sp + u) * r + h] * o8[u];
        }
        for (; sp < nsplit; ++sp) acc += wm[sp * r + h] * load_relaxed(parts + (size_t)sp * row + idx);
        store_out<T>(outp + idx, acc / hz[h]);
    }
}

}  // namespace att
}  // namespace btk
