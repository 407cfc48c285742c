// device_common.hpp -- device helpers of the gfx950 kernels: the Philox
// counter-based generator, the uniform and Gumbel maps, the Markov-bias MFMA
// tile and the partial-result merges.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dspark {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies with the round key bumped by the Weyl constants.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        if (i > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = uint64_t(0xD2511F53u) * c0;
        const uint64_t p1 = uint64_t(0xCD9E8D57u) * c2;
        const uint32_t n0 = uint32_t(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = uint32_t(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = uint32_t(p1);
        c2 = n2;
        c3 = uint32_t(p0);
    }
    return make_uint4(c0, c1, c2, c3);
}

// Counter layout: word0 = (stream << 24) | k, word1 = index i >> 2 (0 for the
// accept stream), word2 = request index, word3 = round id; key = seed.  The
// index i is a vocabulary entry (streams 0, 2) or a 32-entry tile (streams 3,
// 4) and takes output word i & 3.  Stream 0: draft entry noise at position
// k; 1: accept uniform at position k; 2: resample / bonus entry noise at
// position j; 3: draft tile noise; 4: resample / bonus tile noise.
constexpr int kStreamDraft = 0;
constexpr int kStreamAccept = 1;
constexpr int kStreamResample = 2;
constexpr int kStreamDraftTile = 3;
constexpr int kStreamResampleTile = 4;
constexpr int kTile = 32;  // vocabulary entries per tile of the two-level draw

__device__ __forceinline__ uint4 noise_block(int stream, int k, uint32_t vquad, uint32_t req, uint32_t round32,
                                             uint32_t k0, uint32_t k1) {
    return philox4x32_10((uint32_t(stream) << 24) | uint32_t(k), vquad, req, round32, k0, k1);
}

__device__ __forceinline__ uint32_t noise_word(int stream, int k, uint32_t idx, uint32_t req, uint32_t round32,
                                               uint32_t k0, uint32_t k1) {
    const uint4 w = noise_block(stream, k, idx >> 2, req, round32, k0, k1);
    const uint32_t j = idx & 3u;
    return j == 0 ? w.x : (j == 1 ? w.y : (j == 2 ? w.z : w.w));
}

__device__ __forceinline__ uint32_t scalar_word(int stream, int k, uint32_t req, uint32_t round32,
                                                uint32_t k0, uint32_t k1) {
    return philox4x32_10((uint32_t(stream) << 24) | uint32_t(k), 0u, req, round32, k0, k1).x;
}

// u = ((w >> 8) + 0.5) * 2^-24, strictly inside (0, 1).  The value is exact in
// float for u <= 1/2; above 1/2 the odd multiples of 2^-25 are rounded to the
// float grid (an error of at most 2^-25).
__device__ __forceinline__ float uniform01(uint32_t w) {
    return __builtin_fmaf(float(w >> 8), 0x1p-24f, 0x1p-25f);
}

// Gumbel noise in base-2 units: -log2(-log2 u).  z*log2(e) + this is a
// strictly increasing function of z + (-ln(-ln u)), so both pick the same argmax.
// The largest Gumbel values come from u next to 1, where neither u (rounded
// to the float grid) nor the hardware log2 (absolute error about half an ulp
// of 1) leaves any relative accuracy in -log2 u.  There d = 1 - u is formed
// exactly from the complemented word and -log2(1 - d) =
// log2(e) (d + d^2/2 + d^3/3 + d^4/4 + ...) is summed directly: for
// d < 2^-5 the truncation error is below 2e-7 relative; above, the hardware
// log2 of u keeps the relative error of -log2 u below 3e-6.
__device__ __forceinline__ float gumbel2(uint32_t w) {
    const float u = uniform01(w);
    const float d = uniform01(~w);  // 1 - u, exact for u > 1/2
    const float ser =
        d * __builtin_fmaf(d, __builtin_fmaf(d, __builtin_fmaf(d, kLog2e / 4.0f, kLog2e / 3.0f), kLog2e / 2.0f),
                           kLog2e);
    const float e2 = d < 0x1p-5f ? ser : -__builtin_amdgcn_logf(u);
    return -__builtin_amdgcn_logf(e2);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- merges
// Log-sum-exp state (max m, sum s of exp2(. - m)), in base-2 units.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == kNegInf) return;  // both empty
    s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
    m = mn;
}

// (best score, index, second score): larger score wins, lower index on ties.
__device__ __forceinline__ void best_merge(float &b, int &i, float &sc, float b2, int i2, float sc2) {
    const float lo = fminf(b, b2);
    sc = fmaxf(fmaxf(sc, sc2), lo);
    if (b2 > b || (b2 == b && i2 < i)) {
        b = b2;
        i = i2;
    }
}

// ---------------------------------------------------------------- MFMA tile
// The Markov bias of a 32 (vocabulary) x 32 (requests) tile:
// C[v][n] = sum_i W2[v0 + v][i] * E[n][i], E[n] = W1[x_prev of request n].
// A operand = W2 rows (MFMA rows m = lane % 32), B operand = E rows (MFMA
// columns n = lane % 32).  The K index a lane feeds is any bijection shared by
// A and B; lanes of half h = lane / 32 take k = 16 s + 8 h + e (bf16) or
// 8 q + 4 h + e (f32).  Lane (n, h) ends up holding, in acc[4 i + j], the
// bias of vocabulary entry v0 + 8 i + 4 h + j for request column n.

template <typename WT, int R>
struct EFrags;

template <int R>
struct EFrags<uint16_t, R> {
    static_assert(R % 16 == 0 && R >= 16 && R <= 256, "bf16 rank");
    static constexpr int S = R / 16;
    uint4 e[S];
    __device__ __forceinline__ void load(const uint16_t *row, int h) {
#pragma unroll
        for (int s = 0; s < S; ++s) e[s] = *reinterpret_cast<const uint4 *>(row + 16 * s + 8 * h);
    }
};

template <int R>
struct EFrags<float, R> {
    static_assert(R % 8 == 0 && R >= 16 && R <= 128, "f32 rank");
    static constexpr int Q = R / 8;
    float4 e[Q];
    __device__ __forceinline__ void load(const float *row, int h) {
#pragma unroll
        for (int q = 0; q < Q; ++q) e[q] = *reinterpret_cast<const float4 *>(row + 8 * q + 4 * h);
    }
};

template <int R>
__device__ __forceinline__ f32x16_t bias_tile(const EFrags<uint16_t, R> &ef, const uint16_t *w2row, int h) {
    f32x16_t acc = {};
#pragma unroll
    for (int s = 0; s < EFrags<uint16_t, R>::S; ++s) {
        const uint4 a = *reinterpret_cast<const uint4 *>(w2row + 16 * s + 8 * h);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, ef.e[s]), acc, 0, 0, 0);
    }
    return acc;
}

template <int R>
__device__ __forceinline__ f32x16_t bias_tile(const EFrags<float, R> &ef, const float *w2row, int h) {
    f32x16_t acc = {};
#pragma unroll
    for (int q = 0; q < EFrags<float, R>::Q; ++q) {
        const float4 a = *reinterpret_cast<const float4 *>(w2row + 8 * q + 4 * h);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, ef.e[q].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, ef.e[q].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, ef.e[q].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, ef.e[q].w, acc, 0, 0, 0);
    }
    return acc;
}

// W2 tile staged in LDS.  A tile is the 32 rows v0 .. v0 + 31 of W2, RB bytes
// each (RB = r * element size), split into CPR = RB / 16 chunks of 16 bytes.
// Row m's logical chunk c sits in physical chunk c ^ (m & (CPR - 1)), so the
// 32 rows an MFMA fragment read touches at one chunk index fall in distinct
// banks.  The tile is filled by direct global-to-LDS loads: each wave
// instruction writes 64 consecutive 16-byte slots, lane i the i-th, and every
// lane fetches the global chunk that belongs in its slot.
template <typename WT, int R>
struct TileLDS {
    static constexpr int RB = R * int(sizeof(WT));
    static constexpr int CPR = RB / 16;
    static constexpr int BYTES = kTile * RB;
    static constexpr int SLOTS = kTile * CPR;
    static_assert((CPR & (CPR - 1)) == 0 && SLOTS % 64 == 0, "tile layout");
};

// Issue the loads of W2 rows v0 .. v0 + 31 (clamped to V - 1) into `buf`;
// `nthreads` threads of the workgroup take part.
template <typename WT, int R>
__device__ __forceinline__ void tile_issue(const WT *W2, int v0, int V, uint8_t *buf, int nthreads) {
    using L = TileLDS<WT, R>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int s0 = wave * 64; s0 < L::SLOTS; s0 += nthreads) {
        const int slot = s0 + lane;
        const int m = slot / L::CPR;
        const int c = (slot % L::CPR) ^ (m & (L::CPR - 1));
        const int vrow = min(v0 + m, V - 1);
        const uint8_t *g = reinterpret_cast<const uint8_t *>(W2) + size_t(vrow) * L::RB + c * 16;
        __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(buf + s0 * 16),
                                         16, 0, 0);
    }
}

// The Markov-bias MFMA tile with the A operand (W2 rows) read from an LDS tile.
template <int R>
__device__ __forceinline__ f32x16_t bias_tile_lds(const EFrags<uint16_t, R> &ef, const uint8_t *buf, int lane) {
    using L = TileLDS<uint16_t, R>;
    const int m = lane & 31, h = lane >> 5;
    const uint8_t *row = buf + m * L::RB;
    f32x16_t acc = {};
#pragma unroll
    for (int s = 0; s < EFrags<uint16_t, R>::S; ++s) {
        const int c = (2 * s + h) ^ (m & (L::CPR - 1));
        const uint4 a = *reinterpret_cast<const uint4 *>(row + c * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, ef.e[s]), acc, 0, 0, 0);
    }
    return acc;
}

template <int R>
__device__ __forceinline__ f32x16_t bias_tile_lds(const EFrags<float, R> &ef, const uint8_t *buf, int lane) {
    using L = TileLDS<float, R>;
    const int m = lane & 31, h = lane >> 5;
    const uint8_t *row = buf + m * L::RB;
    f32x16_t acc = {};
#pragma unroll
    for (int q = 0; q < EFrags<float, R>::Q; ++q) {
        const int c = (2 * q + h) ^ (m & (L::CPR - 1));
        const float4 a = *reinterpret_cast<const float4 *>(row + c * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, ef.e[q].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, ef.e[q].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, ef.e[q].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, ef.e[q].w, acc, 0, 0, 0);
    }
    return acc;
}

// One Markov-bias entry sum_i W1[prev][i] W2[v][i] on the vector ALUs, split
// over the two lane halves: half h sums i in [h R/2, (h+1) R/2); the halves'
// sums are added with a lane swap.  Used for the within-tile second level.
template <typename WT, int R>
__device__ __forceinline__ float bias_entry(const WT *W1row, const WT *W2row, int h) {
    float d = 0.f;
    constexpr int HALF = R / 2;
    if constexpr (sizeof(WT) == 2) {
#pragma unroll
        for (int q = 0; q < HALF / 8; ++q) {
            const uint4 a = *reinterpret_cast<const uint4 *>(W1row + h * HALF + 8 * q);
            const uint4 w = *reinterpret_cast<const uint4 *>(W2row + h * HALF + 8 * q);
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d = __builtin_fmaf(__uint_as_float(av[e] << 16), __uint_as_float(wv[e] << 16), d);
                d = __builtin_fmaf(__uint_as_float(av[e] & 0xFFFF0000u), __uint_as_float(wv[e] & 0xFFFF0000u), d);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < HALF / 4; ++q) {
            const float4 a = *reinterpret_cast<const float4 *>(W1row + h * HALF + 4 * q);
            const float4 w = *reinterpret_cast<const float4 *>(W2row + h * HALF + 4 * q);
            d = __builtin_fmaf(a.x, w.x, d);
            d = __builtin_fmaf(a.y, w.y, d);
            d = __builtin_fmaf(a.z, w.z, d);
            d = __builtin_fmaf(a.w, w.w, d);
        }
    }
    return d + __shfl_xor(d, 32);
}

// Four consecutive logits starting at v (v % 4 == 0); entries at or past V read
// as -inf.  `vec` says the row allows aligned 16-byte loads.
__device__ __forceinline__ float4 load4_masked(const float *row, int v, int V, bool vec) {
    if (vec && v + 3 < V) return *reinterpret_cast<const float4 *>(row + v);
    float4 r;
    r.x = (v + 0 < V) ? row[v + 0] : kNegInf;
    r.y = (v + 1 < V) ? row[v + 1] : kNegInf;
    r.z = (v + 2 < V) ? row[v + 2] : kNegInf;
    r.w = (v + 3 < V) ? row[v + 3] : kNegInf;
    return r;
}

// The 16 entries of a row that lane half h holds in tile t: t*32 + 8i + 4h + j
// (entries at or past V read as -inf).
__device__ __forceinline__ void load_tile_row(const float *row, int t, int h, int V, bool vec, float4 out[4]) {
    const int v0 = t * kTile;
    if (vec && v0 + kTile <= V) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = *reinterpret_cast<const float4 *>(row + v0 + 8 * i + 4 * h);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = load4_masked(row, v0 + 8 * i + 4 * h, V, vec);
    }
}

__device__ __forceinline__ float f4get(const float4 &a, int j) {
    return j == 0 ? a.x : (j == 1 ? a.y : (j == 2 ? a.z : a.w));
}

__device__ __forceinline__ uint32_t u4get(const uint4 &a, int j) {
    return j == 0 ? a.x : (j == 1 ? a.y : (j == 2 ? a.z : a.w));
}

// Workgroup index remapped so that consecutive logical groups share one XCD:
// the hardware deals workgroups round-robin over the 8 XCDs of the chip.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    constexpr int X = 8;
    const int per = n / X, rem = n % X;
    const int xcd = b % X, pos = b / X;
    return xcd < rem ? xcd * (per + 1) + pos : rem * (per + 1) + (xcd - rem) * per + pos;
}

}  // namespace dspark
