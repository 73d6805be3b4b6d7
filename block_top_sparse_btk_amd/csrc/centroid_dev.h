// Device code of S1 (block centroid = mean of a page's valid keys, fp32
// accumulation), shared by the stand-alone centroid kernel and the
// single-launch decode step.  (Pith review of "Kinetics: Rethinking Test-Time
// Scaling Laws", "What carries the argument": blocks are summarised by their
// averaged key vectors.)
#pragma once
#include "btk_internal.h"

namespace btk {

// Elements of T in one 16-byte vector.
template <typename T>
struct Vec16 {
    static constexpr int n = 16 / (int)sizeof(T);
};

// Mean of the v valid keys of one token-major (page, head) tile, by one wave.
// A key row of D elements is read as 16-byte vectors: LPR lanes cover a token
// row and TPI rows are read per instruction (1 KiB contiguous per wave
// instruction); partial sums over rows are folded with xor shuffles.  The
// loads (KeyTile::load) and the sum (KeyTile::mean) are separate so that a
// caller can put other work between them; the centroid row is written to gdst
// (global) and, if given, to ldst (LDS).
template <typename T, int D>
struct KeyTile {
    static constexpr int VEC = Vec16<T>::n;
    static constexpr int LPR = D / VEC;      // lanes per token row
    static constexpr int TPI = kWave / LPR;  // token rows per wave instruction
    static constexpr int NI = kPage / TPI;   // instructions per tile
    static_assert(kWave % LPR == 0 && kPage % TPI == 0, "layout");
    u32x4_t w[NI];  // raw 16-byte vectors, zero for tokens >= v

    __device__ __forceinline__ void load(const T *tile, int v, int lane) {
        const int col = lane % LPR, row = lane / LPR;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int t = i * TPI + row;
            w[i] = t < v ? *reinterpret_cast<const u32x4_t *>(tile + (size_t)t * D + col * VEC)
                         : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    // token t's row, given as this lane's 16-byte slice (dims col*VEC ..)
    __device__ __forceinline__ void set_row(int t, u32x4_t slice, int lane) {
        const int row = lane / LPR;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (i * TPI + row == t) w[i] = slice;
    }
    // The mean of the v valid rows to gdst (global) and, when ldst is not NULL,
    // to ldst (LDS, the caller's copy; the test is made on a flag because the
    // compiler folded a NULL test of an LDS pointer into an operand form that
    // gfx950 does not encode).
    __device__ __forceinline__ void mean(int v, float *gdst, float *ldst, int lane) const {
        mean_to(v, gdst, ldst, ldst != nullptr, lane);
    }
    __device__ __forceinline__ void mean_to(int v, float *gdst, float *ldst, bool to_lds,
                                            int lane) const {
        const int col = lane % LPR, row = lane / LPR;
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (i * TPI + row < v) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] += vec16_elem<T>(w[i], e);
            }
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
        }
        if (row == 0) {
            const float vf = (float)v;
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const floatx4_t o = {acc[e] / vf, acc[e + 1] / vf, acc[e + 2] / vf,
                                     acc[e + 3] / vf};
                *reinterpret_cast<floatx4_t *>(gdst + col * VEC + e) = o;
                if (to_lds) *reinterpret_cast<floatx4_t *>(ldst + col * VEC + e) = o;
            }
        }
    }
};

template <typename T, int D>
__device__ __forceinline__ void block_centroid(const T *tile, int v, float *gdst, float *ldst,
                                               int lane) {
    KeyTile<T, D> kt;
    kt.load(tile, v, lane);
    kt.mean(v, gdst, ldst, lane);
}

}  // namespace btk
