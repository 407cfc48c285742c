// stage.hpp -- building blocks of the LDS-staged vocabulary walks (draft
// step, resample draw): two-tile stages of W2 rows and logit rows moved into
// LDS by direct loads, and the per-lane tile race.
#pragma once

#include "device_common.hpp"

namespace dspark {

// Cache policy of the direct loads of logit rows (U_k, target rows): they are
// read once a round, so they go in as non-temporal and leave the caches to
// the W2 rows and gathered W1 rows the walks reuse (measured at the headline
// size, with each round's inputs last touched two rounds before: the draft
// step 2.1 us and the draw 4.3 us faster).  W2 tiles keep the default policy.
constexpr int kStreamPolicy = 2;  // the non-temporal bit of the load's cache policy

// Race state of one lane over the tiles it owns: running base-2 logsumexp as
// (max, sum of 2^(z - max)), and the best and second tile scores.
struct TileRace {
    float m, s, best, second;
    int bt;
};

// Scores one 32-entry tile held by this lane in (a, b) (logits U + B, -inf past
// the row end).  Sampled: the tile's logsumexp of z = logit * sc plus its
// Gumbel noise g; greedy: the tile's largest logit.  The sum is taken against
// the running maximum, so one rescale per tile keeps the row total.
template <bool TRACK2>
__device__ __forceinline__ void race_tile(TileRace &st, const f32x16_t &a, const f32x16_t &b, float sc, bool sampled,
                                          int t, float g) {
    float ma = max3f(a[0], a[1], a[2]), mb = max3f(b[0], b[1], b[2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) {
        ma = max3f(ma, a[e], a[e + 1]);
        mb = max3f(mb, b[e], b[e + 1]);
    }
    const float mx = max3f(max3f(ma, a[15], b[15]), mb, mb);
    const float mt = mx * sc;
    const float mn = fmaxf(st.m, mt);
    const float mg = (mn == kNegInf) ? 0.f : mn;
    const float nmg = -mg;
    float s0 = fast_exp2(__builtin_fmaf(a[0], sc, nmg)), s1 = fast_exp2(__builtin_fmaf(a[1], sc, nmg));
    float s2 = fast_exp2(__builtin_fmaf(b[0], sc, nmg)), s3 = fast_exp2(__builtin_fmaf(b[1], sc, nmg));
#pragma unroll
    for (int e = 2; e < 16; e += 2) {
        s0 += fast_exp2(__builtin_fmaf(a[e], sc, nmg));
        s1 += fast_exp2(__builtin_fmaf(a[e + 1], sc, nmg));
        s2 += fast_exp2(__builtin_fmaf(b[e], sc, nmg));
        s3 += fast_exp2(__builtin_fmaf(b[e + 1], sc, nmg));
    }
    const float sum = (s0 + s1) + (s2 + s3);
    st.s = __builtin_fmaf(st.s, fast_exp2(st.m - mg), sum);
    st.m = mn;
    const float Lt = sampled ? mg + fast_log2(sum) + g : mt;
    if (TRACK2) st.second = fmaxf(st.second, fminf(Lt, st.best));
    if (Lt > st.best) {
        st.best = Lt;
        st.bt = t;
    }
}

// Direct-to-LDS loads of one two-tile stage (64 W2 rows) by the workgroup's
// NT threads.  Each thread's slots are fixed, so their source offsets are
// computed once.
template <typename WT, int R, int NT>
struct StageDMA {
    using L = TileLDS<WT, R>;
    static constexpr int SLOTS = 2 * L::SLOTS;  // 16-byte slots of a stage
    static constexpr int J = (SLOTS + NT - 1) / NT;
    // load instructions every wave issues a stage (the last waves may issue
    // fewer than J when a stage has fewer slots than the workgroup threads)
    static constexpr int MIN_PER_WAVE = SLOTS > NT - 64 ? (SLOTS - (NT - 64) - 1) / NT + 1 : 0;
    uint32_t goff[J];  // byte offset of the slot's source from the stage's first row
    int row[J];        // stage row (0..63) the slot belongs to

    __device__ __forceinline__ void init(int tid) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int slot = tid + j * NT;
            const int m = slot / L::CPR;
            row[j] = m;
            goff[j] = uint32_t(m * L::RB + L::chunk(m, slot % L::CPR) * 16);
        }
    }
    // rows v0 .. v0 + 63; CLAMP repeats row V - 1 for rows past the vocabulary
    template <bool CLAMP>
    __device__ __forceinline__ void issue(const WT *W2, int v0, int V, uint8_t *buf, int wave) const {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(W2) + size_t(v0) * L::RB;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int s0 = wave * 64 + j * NT;  // slot of lane 0, uniform
            if (J * NT > SLOTS && s0 >= SLOTS) break;
            const uint8_t *g = src + goff[j];
            if (CLAMP) {
                const int vrow = min(v0 + row[j], V - 1);
                g = reinterpret_cast<const uint8_t *>(W2) + size_t(vrow) * L::RB + (goff[j] - uint32_t(row[j] * L::RB));
            }
            __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(buf + s0 * 16), 16, 0, 0);
        }
    }
};

// The logit rows of a two-tile stage for one wave's 32 requests: 32 rows of
// 64 floats, staged in a wave-private LDS region by direct loads so that each
// load instruction covers whole 256-byte row segments, then read back in the
// MFMA accumulator layout.  In LDS the 16-byte chunk c of row r sits at chunk
// c ^ (r & 15).  VEC moves 16 bytes a lane (rows allow aligned 16-byte
// loads), else 4 bytes.
template <bool VEC>
struct StageRows {
    static constexpr int ROWB = 2 * kTile * 4;          // bytes of a row segment
    static constexpr int BYTES = 32 * ROWB;             // one wave's region
    static constexpr int NI = VEC ? BYTES / 1024 : BYTES / 256;  // load instructions a stage
    const float *base;  // region row r reads base + idx * stride
    size_t stride;
    int idx[NI];        // source row of each instruction's lane

    // row(r) is the source row index of region row r (0..31); every region
    // row has one, so that a stage is always NI load instructions a lane
    template <typename RowFn>
    __device__ __forceinline__ void init(int lane, const float *base_, size_t stride_, RowFn row) {
        base = base_;
        stride = stride_;
#pragma unroll
        for (int j = 0; j < NI; ++j) idx[j] = row(region_row(j, lane));
    }
    __device__ static __forceinline__ int region_row(int j, int lane) { return VEC ? 4 * j + (lane >> 4) : j; }
    // first column (relative to the stage) of the lane's 16 (or 4) bytes
    __device__ static __forceinline__ int region_col(int j, int lane) {
        const int r = region_row(j, lane);
        return VEC ? 4 * ((lane & 15) ^ (r & 15)) : 4 * (((lane >> 2) ^ r) & 15) + (lane & 3);
    }
    template <bool CLAMP>
    __device__ __forceinline__ void issue(int v0, int V, uint8_t *region, int lane) const {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            int v = v0 + region_col(j, lane);
            if (CLAMP) v = min(v, V - (VEC ? 4 : 1));
            const void *g = base + size_t(idx[j]) * stride + v;
            if constexpr (VEC)
                __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(region + j * 1024), 16, 0,
                                                 kStreamPolicy);
            else
                __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(region + j * 256), 4, 0,
                                                 kStreamPolicy);
        }
    }
    // accumulator layout: value 4i+j of lane (n, h) is entry 32q + 8i + 4h + j
    __device__ __forceinline__ void read(const uint8_t *region, int lane, f32x16_t &c0, f32x16_t &c1) const {
        const int n = lane & 31, h = lane >> 5;
        const uint8_t *row = region + n * ROWB;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f32x16_t &c = q ? c1 : c0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = (8 * q + 2 * i + h) ^ (n & 15);
                const float4 x = *reinterpret_cast<const float4 *>(row + ch * 16);
                c[4 * i] = x.x;
                c[4 * i + 1] = x.y;
                c[4 * i + 2] = x.z;
                c[4 * i + 3] = x.w;
            }
        }
    }
    // the lane-half-swapped layout: lane (n, h) gets tile h of the stage for
    // row n, entries 8i+j in c0[4i+j] and 8i+4+j in c1[4i+j]
    __device__ __forceinline__ void read_swapped(const uint8_t *region, int lane, f32x16_t &c0, f32x16_t &c1) const {
        const int n = lane & 31, h = lane >> 5;
        const uint8_t *row = region + n * ROWB;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            f32x16_t &c = (k & 1) ? c1 : c0;
            const int i = k >> 1;
            const float4 x = *reinterpret_cast<const float4 *>(row + (((8 * h + k) ^ (n & 15)) * 16));
            c[4 * i] = x.x;
            c[4 * i + 1] = x.y;
            c[4 * i + 2] = x.z;
            c[4 * i + 3] = x.w;
        }
    }
};

// The logit rows of a one-tile stage for one wave's 32 requests: 32 rows of
// 32 floats in a wave-private LDS region, loaded by direct loads (each load
// instruction covers whole 128-byte row segments) and read back in the MFMA
// accumulator layout.  In LDS the 16-byte chunk c of row r sits at chunk
// c ^ (r & 7).  VEC moves 16 bytes a lane, else 4 bytes.
template <bool VEC>
struct TileRows {
    static constexpr int ROWB = kTile * 4;                      // bytes of a row segment
    static constexpr int BYTES = 32 * ROWB;                     // one wave's region
    static constexpr int NI = VEC ? BYTES / 1024 : BYTES / 256;  // load instructions a stage
    const float *base;  // region row r reads base + idx * stride
    size_t stride;
    int idx[NI];        // source row of each instruction's lane, -1 for none

    __device__ static __forceinline__ int region_row(int j, int lane) { return VEC ? 8 * j + (lane >> 3) : 2 * j + (lane >> 5); }
    __device__ static __forceinline__ int region_col(int j, int lane) {
        const int r = region_row(j, lane);
        return VEC ? 4 * ((lane & 7) ^ (r & 7)) : 4 * (((lane >> 2) & 7) ^ (r & 7)) + (lane & 3);
    }
    template <typename RowFn>
    __device__ __forceinline__ void init(int lane, const float *base_, size_t stride_, RowFn row) {
        base = base_;
        stride = stride_;
#pragma unroll
        for (int j = 0; j < NI; ++j) idx[j] = row(region_row(j, lane));
    }
    // rows without a source are skipped (their region rows keep stale data)
    template <bool CLAMP>
    __device__ __forceinline__ void issue(int v0, int V, uint8_t *region, int lane) const {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            int v = v0 + region_col(j, lane);
            if (CLAMP) v = min(v, V - (VEC ? 4 : 1));
            if (idx[j] < 0) continue;
            const void *g = base + size_t(idx[j]) * stride + v;
            if constexpr (VEC)
                __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(region + j * 1024), 16, 0,
                                                 kStreamPolicy);
            else
                __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(region + j * 256), 4, 0,
                                                 kStreamPolicy);
        }
    }
    // accumulator layout: value 4i+j of lane (n, h) is entry 8i + 4h + j
    __device__ __forceinline__ f32x16_t read(const uint8_t *region, int lane) const {
        const int n = lane & 31, h = lane >> 5;
        const uint8_t *row = region + n * ROWB;
        f32x16_t c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 x = *reinterpret_cast<const float4 *>(row + (((2 * i + h) ^ (n & 7)) * 16));
            c[4 * i] = x.x;
            c[4 * i + 1] = x.y;
            c[4 * i + 2] = x.z;
            c[4 * i + 3] = x.w;
        }
        return c;
    }
};

// Direct-to-LDS loads of one tile (32 W2 rows) by the workgroup's NT threads,
// with the per-thread source offsets computed once.
template <typename WT, int R, int NT>
struct TileDMA {
    using L = TileLDS<WT, R>;
    static constexpr int J = (L::SLOTS + NT - 1) / NT;
    uint32_t goff[J];
    int row[J];

    __device__ __forceinline__ void init(int tid) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int slot = tid + j * NT;
            const int m = slot / L::CPR;
            row[j] = m;
            goff[j] = uint32_t(m * L::RB + L::chunk(m, slot % L::CPR) * 16);
        }
    }
    template <bool CLAMP>
    __device__ __forceinline__ void issue(const WT *W2, int v0, int V, uint8_t *buf, int wave) const {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(W2) + size_t(v0) * L::RB;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int s0 = wave * 64 + j * NT;  // slot of lane 0, uniform
            if (J * NT > L::SLOTS && s0 >= L::SLOTS) break;
            const uint8_t *g = src + goff[j];
            if (CLAMP) {
                const int vrow = min(v0 + row[j], V - 1);
                g = reinterpret_cast<const uint8_t *>(W2) + size_t(vrow) * L::RB + (goff[j] - uint32_t(row[j] * L::RB));
            }
            __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(buf + s0 * 16), 16, 0, 0);
        }
    }
};

}  // namespace dspark
