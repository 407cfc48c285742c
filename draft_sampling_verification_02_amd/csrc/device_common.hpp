// device_common.hpp -- device helpers of the gfx950 kernels: the Philox
// counter-based generator, the uniform and Gumbel maps, the Markov-bias MFMA
// tile and the partial-result merges.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace dspark {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

// v_max3_f32, without the NaN-quieting self-max that IEEE mode makes the
// compiler put in front of every fmaxf of a loaded or exchanged value.
// Inline asm is opaque to the compiler's hazard tracking, so its operands must
// come from ordinary VALU or memory instructions, never straight from an MFMA
// accumulator (the required wait states after the MFMA would be missing).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
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

// ---------------------------------------------------------------- butterflies
// The partner value of a 64-lane all-reduce at step S, on the vector ALUs
// (no round trip through the LDS crossbar).  Step 0 pairs lane i with i ^ 1
// and step 1 with i ^ 2 (quad permutes), step 2 with 7 - i within its group
// of 8 (row half mirror), step 3 with 15 - i within its row of 16 (row
// mirror), step 4 with i ^ 16 and step 5 with i ^ 32 (v_permlane16_swap and
// v_permlane32_swap of x with itself, which hand each row or half its
// partner's copy).  Each step joins two groups that earlier steps have
// already reduced, so after steps 0..3 every lane holds its row's result,
// after step 4 its half's and after step 5 the wave's.  Every lane of the
// wave must be active.
template <int S>
__device__ __forceinline__ uint32_t bfly_u32(uint32_t x) {
    if constexpr (S == 0) {
        return uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    } else if constexpr (S == 1) {
        return uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    } else if constexpr (S == 2) {
        return uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    } else if constexpr (S == 3) {
        return uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x140, 0xF, 0xF, false));  // row_mirror
    } else if constexpr (S == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (threadIdx.x & 16) ? r[0] : r[1];
    } else {
        static_assert(S == 5, "six steps");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (threadIdx.x & 32) ? r[0] : r[1];
    }
}
template <int S>
__device__ __forceinline__ float bfly(float x) {
    return __uint_as_float(bfly_u32<S>(__float_as_uint(x)));
}
template <int S>
__device__ __forceinline__ int bfly(int x) {
    return int(bfly_u32<S>(uint32_t(x)));
}
// f(std::integral_constant<int, S>) for S = S0 .. S1 - 1, in order
template <int S0, int S1, class F>
__device__ __forceinline__ void bfly_steps(F &&f) {
    if constexpr (S0 < S1) {
        f(std::integral_constant<int, S0>{});
        bfly_steps<S0 + 1, S1>(f);
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
    // from a packed block (PackedE): one 1 KiB contiguous load a fragment
    __device__ __forceinline__ void load_packed(const uint4 *blk, int lane) {
#pragma unroll
        for (int s = 0; s < S; ++s) e[s] = blk[s * 64 + lane];
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int s = 0; s < S; ++s) e[s] = make_uint4(0u, 0u, 0u, 0u);
    }
    // the fragments as values an empty asm defines (waits for their loads)
    __device__ __forceinline__ void pin() {
#pragma unroll
        for (int s = 0; s < S; ++s) asm volatile("" : "+v"(e[s].x), "+v"(e[s].y), "+v"(e[s].z), "+v"(e[s].w));
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
    __device__ __forceinline__ void load_packed(const uint4 *blk, int lane) {
#pragma unroll
        for (int q = 0; q < Q; ++q) e[q] = reinterpret_cast<const float4 *>(blk)[q * 64 + lane];
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int q = 0; q < Q; ++q) e[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ void pin() {
#pragma unroll
        for (int q = 0; q < Q; ++q) asm volatile("" : "+v"(e[q].x), "+v"(e[q].y), "+v"(e[q].z), "+v"(e[q].w));
    }
};

// W2 tile staged in LDS.  A tile is the 32 rows v0 .. v0 + 31 of W2, RB bytes
// each (RB = r * element size), split into CPR = RB / 16 chunks of 16 bytes.
// Within each group of SW = min(CPR, 16) chunks, row m's logical chunk c sits
// at c ^ (m & (SW - 1)), so the rows an MFMA fragment read touches at one
// chunk index fall in distinct banks.  The tile is filled by direct
// global-to-LDS loads: each wave instruction writes 64 consecutive 16-byte
// slots, lane i the i-th, and every lane fetches the global chunk that
// belongs in its slot.
template <typename WT, int R>
struct TileLDS {
    static constexpr int RB = R * int(sizeof(WT));
    static constexpr int CPR = RB / 16;
    static constexpr int BYTES = kTile * RB;
    static constexpr int SLOTS = kTile * CPR;
    static constexpr int SW = CPR < 16 ? CPR : 16;  // chunks per swizzle group
    static_assert((CPR & (CPR - 1)) == 0 && SLOTS % 64 == 0, "tile layout");
    // physical 16-byte chunk of logical chunk c of row m: the low bits of c are
    // XORed with the row, so the rows that one LDS cycle serves hit distinct banks
    __device__ static __forceinline__ int chunk(int m, int c) { return (c & ~(SW - 1)) | ((c ^ m) & (SW - 1)); }
};

// The Markov-bias MFMA tile with the A operand (W2 rows) read from an LDS tile.
template <int R>
__device__ __forceinline__ f32x16_t bias_tile_lds(const EFrags<uint16_t, R> &ef, const uint8_t *buf, int lane,
                                                  f32x16_t acc = {}) {
    using L = TileLDS<uint16_t, R>;
    const int m = lane & 31, h = lane >> 5;
    const uint8_t *row = buf + m * L::RB;
#pragma unroll
    for (int s = 0; s < EFrags<uint16_t, R>::S; ++s) {
        const uint4 a = *reinterpret_cast<const uint4 *>(row + L::chunk(m, 2 * s + h) * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, ef.e[s]), acc, 0, 0, 0);
    }
    return acc;
}

template <int R>
__device__ __forceinline__ f32x16_t bias_tile_lds(const EFrags<float, R> &ef, const uint8_t *buf, int lane,
                                                  f32x16_t acc = {}) {
    using L = TileLDS<float, R>;
    const int m = lane & 31, h = lane >> 5;
    const uint8_t *row = buf + m * L::RB;
#pragma unroll
    for (int q = 0; q < EFrags<float, R>::Q; ++q) {
        const float4 a = *reinterpret_cast<const float4 *>(row + L::chunk(m, 2 * q + h) * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, ef.e[q].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, ef.e[q].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, ef.e[q].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, ef.e[q].w, acc, 0, 0, 0);
    }
    return acc;
}

// Packed E rows: the B-operand fragments of a block of 32 requests laid out
// in the order the MFMA tile reads them, so that a wave loads each fragment
// with one contiguous 1 KiB instruction.  A row of RB bytes is 2 NF chunks of
// 16 bytes (NF = RB / 32); chunk c of request n's row sits at 16-byte slot
// (f * 64 + n + 32 hh) of its block, f = c / 2, hh = c % 2 (lane (n, hh)
// feeds chunk 2 f + hh at K-step f, as EFrags::load does from the row).
template <typename WT, int R>
struct PackedE {
    static constexpr int NF = R * int(sizeof(WT)) / 32;  // fragments (K-steps) a row
    static constexpr int BLOCK = NF * 64;                 // 16-byte slots a block of 32 requests
    __device__ static __forceinline__ int slot(int n, int c) { return (c >> 1) * 64 + n + 32 * (c & 1); }
};

// One lane half's share of a W1 row (entries [h * R/2, (h + 1) * R/2)) held
// in registers, and its dot product with the same share of a W2 row.
template <typename WT, int R>
struct RowHalf {
    static constexpr int HALF = R / 2;
    static constexpr int N = HALF * int(sizeof(WT)) / 16;  // 16-byte pieces
    uint4 w[N];
    __device__ __forceinline__ void load(const WT *row, int h) {
        const uint4 *q = reinterpret_cast<const uint4 *>(row + h * HALF);
#pragma unroll
        for (int i = 0; i < N; ++i) w[i] = q[i];
    }
    // this half of the row into row n of a PackedE block: piece i is chunk
    // h N + i of the row
    __device__ __forceinline__ void store_packed(uint4 *blk, int n, int h) const {
#pragma unroll
        for (int i = 0; i < N; ++i) blk[PackedE<WT, R>::slot(n, h * N + i)] = w[i];
    }
    // the full dot product W1row . W2row, summed over the two lane halves:
    // four independent accumulator chains, bf16 pairs through v_dot2 (each
    // bf16 product is exact in fp32)
    __device__ __forceinline__ float dot(const WT *W2row, int h) const {
        const uint4 *q = reinterpret_cast<const uint4 *>(W2row + h * HALF);
        uint4 x[N];
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = q[i];
        float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t av[4] = {w[i].x, w[i].y, w[i].z, w[i].w}, xv[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (sizeof(WT) == 2) {
                    d[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[e]),
                                                           __builtin_bit_cast(bf16x2_t, xv[e]), d[e], false);
                } else {
                    d[e] = __builtin_fmaf(__uint_as_float(av[e]), __uint_as_float(xv[e]), d[e]);
                }
            }
        }
        const float t = (d[0] + d[1]) + (d[2] + d[3]);
        return t + bfly<5>(t);
    }
};

// The 32 dot products e . row(m), m = 0..31, of a tile of rows of R entries
// (W2 rows of a vocabulary tile), read in whole lines: load instruction j of
// the wave covers 1 KiB of the tile, lane l the 16-byte chunk c = l % CPR of
// row RPI j + l / CPR.  Each lane dots its chunks with chunk c of e (one
// 16-byte piece a lane), then a transposing butterfly over the CPR lanes of a
// row group sums every row: at the step on lane bit b (highest first) each
// lane keeps the half of its remaining rows that bit b selects and adds its
// partner's sums for them (the partner flips bit b and agrees on every bit
// already taken, so the mirror permutes serve too).  Lane l ends up with the
// full sum of row RPI (c >> 1) + l / CPR; lanes l and l ^ 1 hold the same row.
template <typename WT, int R>
struct TileDot {
    static constexpr int RB = R * int(sizeof(WT));
    static constexpr int CPR = RB / 16;               // 16-byte chunks a row
    static constexpr int NI = CPR / 2 > 0 ? CPR / 2 : 1;  // load instructions a tile
    static constexpr int RPI = 64 / CPR;              // rows an instruction covers
    static_assert(CPR >= 2 && CPR <= 32 && (CPR & (CPR - 1)) == 0, "tile row size");
    uint4 w[NI];
    __device__ static __forceinline__ int row_of(int lane) { return RPI * ((lane % CPR) >> 1) + lane / CPR; }
    __device__ static __forceinline__ int lane_of(int m) { return (m % RPI) * CPR + 2 * (m / RPI); }
    // rows v0 .. v0 + 31 of M (row stride R), rows past vmax repeat row vmax
    __device__ __forceinline__ void load(const WT *M, int v0, int vmax, int lane) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int v = min(v0 + RPI * j + lane / CPR, vmax);
            w[j] = reinterpret_cast<const uint4 *>(M + size_t(v) * R)[lane % CPR];
        }
    }
    __device__ static __forceinline__ float chunk_dot(const uint4 &a, const uint4 &e) {
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, ev[4] = {e.x, e.y, e.z, e.w};
        float d0 = 0.f, d1 = 0.f;
        if constexpr (sizeof(WT) == 2) {
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[0]), __builtin_bit_cast(bf16x2_t, ev[0]),
                                                 d0, false);
            d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[1]), __builtin_bit_cast(bf16x2_t, ev[1]),
                                                 d1, false);
            d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[2]), __builtin_bit_cast(bf16x2_t, ev[2]),
                                                 d0, false);
            d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[3]), __builtin_bit_cast(bf16x2_t, ev[3]),
                                                 d1, false);
        } else {
            d0 = __uint_as_float(av[0]) * __uint_as_float(ev[0]);
            d1 = __uint_as_float(av[1]) * __uint_as_float(ev[1]);
            d0 = __builtin_fmaf(__uint_as_float(av[2]), __uint_as_float(ev[2]), d0);
            d1 = __builtin_fmaf(__uint_as_float(av[3]), __uint_as_float(ev[3]), d1);
        }
        return d0 + d1;
    }
    // e: chunk lane % CPR of the vector; every lane of the wave must be active
    __device__ __forceinline__ float dot(const uint4 &e) const {
        float p[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) p[j] = chunk_dot(w[j], e);
        const int lane = threadIdx.x & 63;
        bfly_steps<0, 6>([&](auto st) {
            constexpr int B = 5 - decltype(st)::value;  // lane bit, highest first
            if constexpr ((1 << B) < CPR && B >= 1) {
                constexpr int HALF = 1 << (B - 1);  // rows a lane keeps: 2^B before the step
                const bool up = (lane >> B) & 1;
#pragma unroll
                for (int t = 0; t < HALF; ++t) {
                    const float keep = up ? p[HALF + t] : p[t];
                    const float send = up ? p[t] : p[HALF + t];
                    p[t] = keep + bfly<B>(send);
                }
            }
        });
        return p[0] + bfly<0>(p[0]);
    }
};

// Two C-initialised MFMA chains over the two 32-row tiles of a stage (buf and
// buf + one tile), sharing the E fragments; the A fragments are read from LDS
// a few K-steps ahead of their MFMAs.
template <int R>
__device__ __forceinline__ void bias_pair_lds(const EFrags<uint16_t, R> &ef, const uint8_t *buf, int lane,
                                              f32x16_t &c0, f32x16_t &c1) {
    using L = TileLDS<uint16_t, R>;
    constexpr int S = EFrags<uint16_t, R>::S;
    constexpr int D = S < 3 ? S : 3;  // K-steps in flight
    const int m = lane & 31, h = lane >> 5;
    const uint8_t *row = buf + m * L::RB;
    uint4 a0[D], a1[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        a0[s] = *reinterpret_cast<const uint4 *>(row + L::chunk(m, 2 * s + h) * 16);
        a1[s] = *reinterpret_cast<const uint4 *>(row + L::BYTES + L::chunk(m, 2 * s + h) * 16);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint4 x0 = a0[s % D], x1 = a1[s % D];
        if (s + D < S) {
            a0[s % D] = *reinterpret_cast<const uint4 *>(row + L::chunk(m, 2 * (s + D) + h) * 16);
            a1[s % D] = *reinterpret_cast<const uint4 *>(row + L::BYTES + L::chunk(m, 2 * (s + D) + h) * 16);
        }
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x0),
                                                     __builtin_bit_cast(bf16x8_t, ef.e[s]), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x1),
                                                     __builtin_bit_cast(bf16x8_t, ef.e[s]), c1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads D steps ahead of their MFMAs
    }
}

template <int R>
__device__ __forceinline__ void bias_pair_lds(const EFrags<float, R> &ef, const uint8_t *buf, int lane,
                                              f32x16_t &c0, f32x16_t &c1) {
    using L = TileLDS<float, R>;
    constexpr int Q = EFrags<float, R>::Q;
    constexpr int D = Q < 3 ? Q : 3;
    const int m = lane & 31, h = lane >> 5;
    const uint8_t *row = buf + m * L::RB;
    float4 a0[D], a1[D];
#pragma unroll
    for (int q = 0; q < D; ++q) {
        a0[q] = *reinterpret_cast<const float4 *>(row + L::chunk(m, 2 * q + h) * 16);
        a1[q] = *reinterpret_cast<const float4 *>(row + L::BYTES + L::chunk(m, 2 * q + h) * 16);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const float4 x0 = a0[q % D], x1 = a1[q % D];
        if (q + D < Q) {
            a0[q % D] = *reinterpret_cast<const float4 *>(row + L::chunk(m, 2 * (q + D) + h) * 16);
            a1[q % D] = *reinterpret_cast<const float4 *>(row + L::BYTES + L::chunk(m, 2 * (q + D) + h) * 16);
        }
        const float4 e = ef.e[q];
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0.x, e.x, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1.x, e.x, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0.y, e.y, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1.y, e.y, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0.z, e.z, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1.z, e.z, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0.w, e.w, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1.w, e.w, c1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// x of lane n plus (or max with) x of lane n ^ 32, in every lane: one
// v_permlane32_swap of x with itself hands each half the other half's x.
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Exchange the lane halves of two accumulator tiles (v_permlane32_swap, which
// swaps lanes 32..63 of its first operand with lanes 0..31 of its second).
// Before: lane (n, h) holds rows 8i+4h+j of tile a in a and of tile b in b.
// After: lanes 0..31 hold every row of tile a (a: rows 8i+j, b: rows 8i+4+j)
// and lanes 32..63 every row of tile b, in the same arrangement.
__device__ __forceinline__ void swap_halves(f32x16_t &a, f32x16_t &b) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[e]), __float_as_uint(b[e]), false, false);
        a[e] = __uint_as_float(r[0]);
        b[e] = __uint_as_float(r[1]);
    }
}

__device__ __forceinline__ float f4get(const float4 &a, int j) {
    return j == 0 ? a.x : (j == 1 ? a.y : (j == 2 ? a.z : a.w));
}

__device__ __forceinline__ uint32_t u4get(const uint4 &a, int j) {
    return j == 0 ? a.x : (j == 1 ? a.y : (j == 2 ? a.z : a.w));
}

// A float4 of a logit row that is read once (target rows in the position
// passes and the acceptance statistics): a non-temporal load, which leaves
// the caches to the W2 rows and gathered W1 rows that are reused.
__device__ __forceinline__ float4 load_stream(const float4 *q) {
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(q));
    return make_float4(x.x, x.y, x.z, x.w);
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
