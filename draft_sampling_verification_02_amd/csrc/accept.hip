// accept.hip -- the exact per-position acceptance probability of a verified
// block on gfx950, the confidence head's training label.
//
// Method (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
// section 4.1: under rejection sampling a draft passes with probability one
// minus the total-variation distance of the draft and target distributions;
// "DeepSeek DSpark explained" (share.concentrate1.com), section 05: the
// accepted mass is min(p, q)):
//   alpha_k = sum_v min(p_k(v), q_k(v)),
//   p_k = softmax(t_k / T),  q_k = softmax((U_k + W1[x_{k-1}] W2^T) / T),
// for every verified position k <= ell_b on the drafted prefix.  T = 0: both
// are one-hot (q_k at the greedy draft x_k, p_k at the lowest-index argmax of
// t_k), so alpha_k is 1 when they agree and 0 otherwise.
//
// Kernels, in launch order:
//   accept_prep      1 workgroup: input checks and row offsets (as the verify
//                    half does them), the list of (request, position) rows --
//                    sampled rows first, greedy rows after -- and NaN defaults.
//   accept_rowstats  one workgroup per (listed row, vocabulary segment):
//                    base-2 logsumexp of t / T (sampled rows) or the
//                    lowest-index argmax of t (greedy rows).
//   accept_mass      waves of 32 sampled rows walk vocabulary chunks: the q_k
//                    logits of a tile come from the draft's LDS-staged MFMA
//                    bias tile on top of the staged U_k tile, the target tile
//                    is staged beside it, and each lane sums min(p, q).
//   accept_finish    one thread per listed row: the chunk sums (sampled) or the
//                    argmax match (greedy) into alpha_out.
#include "device_common.hpp"
#include "internal.hpp"
#include "stage.hpp"

#include <algorithm>
#include <type_traits>

namespace dspark {

namespace {

constexpr int kAccThreads = 512;  // accept_mass: 8 waves of 32 listed rows
constexpr int kRowThreads = 256;  // accept_rowstats

// Exclusive scan over a workgroup of NT threads of one int per thread.
template <int NT>
__device__ int acc_block_scan(int v, int *lds, int *total) {
    const int t = threadIdx.x;
    lds[t] = v;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
        const int add = (t >= o) ? lds[t - o] : 0;
        __syncthreads();
        lds[t] += add;
        __syncthreads();
    }
    const int incl = lds[t];
    if (total) *total = lds[NT - 1];
    __syncthreads();
    return incl - v;
}

// ------------------------------------------------------------------ prep

struct AccPrepParams {
    const int32_t *ell, *row_offsets, *anchor, *x;
    const float *temperature;
    int B, gamma, V, n_target_rows;
    int32_t *count;     // [2] sampled rows, greedy rows
    int32_t *ent_rho;   // [B * gamma] row b * gamma + k - 1 of the listed entry
    int32_t *ent_trow;  // packed target row
    int32_t *ent_prev;  // the head's row: x_{k-1}, or b * gamma + k - 1 (erow_mode)
    float *alpha_out;
    int erow_mode;
};

// A request is listed when 0 <= ell_b <= gamma and its rows lie in the target
// (with the caller's offsets: off_0 >= 0 and off_{b+1} - off_b = 1 + ell_b).
__global__ __launch_bounds__(1024) void accept_prep_kernel(AccPrepParams p) {
    __shared__ int lds[1024];
    const int t = threadIdx.x;
    const int seg = (p.B + 1023) / 1024;
    const int b0 = min(p.B, t * seg), b1 = min(p.B, b0 + seg);
    auto clamp_ell = [&](int b) __device__ { return min(max(p.ell[b], 0), p.gamma); };
    // packed offsets of the computed layout
    int local = 0;
    for (int b = b0; b < b1; ++b) local += 1 + clamp_ell(b);
    int base = acc_block_scan<1024>(local, lds, nullptr);
    // which requests are listed, and their row counts by kind
    int ns_local = 0, ng_local = 0;
    {
        int o = base;
        for (int b = b0; b < b1; ++b) {
            const int e_raw = p.ell[b], e = clamp_ell(b);
            bool ok = e_raw == e;
            int off = o;
            if (p.row_offsets) {
                off = p.row_offsets[b];
                if (off < 0 || p.row_offsets[b + 1] - off != 1 + e_raw) ok = false;
            }
            if (ok && off + e + 1 > p.n_target_rows) ok = false;
            if (ok) {
                if (p.temperature[b] > 0.f)
                    ns_local += e;
                else
                    ng_local += e;
            }
            o += 1 + e;
        }
    }
    int ns = 0, ng = 0;
    const int sbase = acc_block_scan<1024>(ns_local, lds, &ns);
    const int gbase = acc_block_scan<1024>(ng_local, lds, &ng);
    int si = sbase, gi = ns + gbase, o = base;
    for (int b = b0; b < b1; ++b) {
        const int e_raw = p.ell[b], e = clamp_ell(b);
        bool ok = e_raw == e;
        int off = o;
        if (p.row_offsets) {
            off = p.row_offsets[b];
            if (off < 0 || p.row_offsets[b + 1] - off != 1 + e_raw) ok = false;
        }
        if (ok && off + e + 1 > p.n_target_rows) ok = false;
        const bool sampled = p.temperature[b] > 0.f;
        for (int k = 1; k <= p.gamma; ++k) {
            const int rho = b * p.gamma + k - 1;
            p.alpha_out[rho] = __builtin_nanf("");
            if (!ok || k > e) continue;
            const int slot = sampled ? si++ : gi++;
            p.ent_rho[slot] = rho;
            p.ent_trow[slot] = off + k - 1;
            const int prev = k == 1 ? p.anchor[b] : p.x[size_t(b) * p.gamma + k - 2];
            p.ent_prev[slot] = p.erow_mode ? rho : min(max(prev, 0), p.V - 1);
        }
        o += 1 + e;
    }
    if (t == 0) {
        p.count[0] = ns;
        p.count[1] = ng;
    }
}

// ------------------------------------------------------------------ row statistics

struct AccRowParams {
    const float *target, *temperature;
    int gamma, V, nseg, seg_len;
    const int32_t *count, *ent_rho, *ent_trow;
    float *rs_m, *rs_s, *rs_v;  // [entries, nseg]
    int32_t *rs_i;
};

// One workgroup per (listed row, segment).  Sampled rows: base-2 logsumexp
// (max, sum of 2^(z - max)) of z = t / T in log2 units; greedy rows: the
// largest t and its lowest index.  Loads are unconditional (clamped into the
// segment and masked after), four 16-byte groups (VEC) or four entries a
// thread per batch.
template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void accept_rowstats_kernel(AccRowParams p) {
    const int e = blockIdx.x / p.nseg, sg = blockIdx.x % p.nseg;
    if (e >= p.count[0] + p.count[1]) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rho = p.ent_rho[e];
    const float T = p.temperature[rho / p.gamma];
    const bool sampled = T > 0.f;
    const float sc = sampled ? kLog2e / T : 1.0f;
    const int v_lo = sg * p.seg_len, v_hi = min(p.V, v_lo + p.seg_len);
    const float *row = p.target + size_t(p.ent_trow[e]) * p.V;
    float m = kNegInf, s = 0.f, av = kNegInf;
    int ai = 0x7fffffff;
    auto walk = [&](auto argmax_c) __device__ {
        constexpr bool ARGMAX = decltype(argmax_c)::value;
        constexpr int W = VEC ? 4 : 1;                 // entries a load
        constexpr int STEP = W * kRowThreads * 4;      // entries a batch
        for (int v0 = v_lo + W * tid; v0 < v_hi; v0 += STEP) {
            float x[4][W];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = min(v0 + W * kRowThreads * u, v_hi - W);
                if constexpr (VEC) {
                    const float4 q = load_stream(reinterpret_cast<const float4 *>(row + v));
                    x[u][0] = q.x;
                    x[u][1] = q.y;
                    x[u][2] = q.z;
                    x[u][3] = q.w;
                } else {
                    x[u][0] = row[v];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = v0 + W * kRowThreads * u < v_hi;
#pragma unroll
                for (int j = 0; j < W; ++j) x[u][j] = ok ? x[u][j] : kNegInf;
            }
            if constexpr (ARGMAX) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < W; ++j)
                        if (x[u][j] > av) {
                            av = x[u][j];
                            ai = v0 + W * kRowThreads * u + j;
                        }
            } else {
                float bm = x[0][0];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < W; ++j) bm = fmaxf(bm, x[u][j]);
                const float nm = fmaxf(m, bm * sc);
                const float mg = nm == kNegInf ? 0.f : nm;
                float add = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < W; ++j) add += fast_exp2(__builtin_fmaf(x[u][j], sc, -mg));
                s = __builtin_fmaf(s, fast_exp2(m - mg), add);
                m = nm;
            }
        }
    };
    if (sampled)
        walk(std::integral_constant<bool, false>{});
    else
        walk(std::integral_constant<bool, true>{});
    // workgroup merge: the wave, then the four waves through LDS
    bfly_steps<0, 6>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float m2 = bfly<S>(m), s2 = bfly<S>(s), v2 = bfly<S>(av);
        const int i2 = bfly<S>(ai);
        lse_merge(m, s, m2, s2);
        if (v2 > av || (v2 == av && i2 < ai)) {
            av = v2;
            ai = i2;
        }
    });
    __shared__ float lm[4], ls[4], lv[4];
    __shared__ int li[4];
    if (lane == 0) {
        lm[wave] = m;
        ls[wave] = s;
        lv[wave] = av;
        li[wave] = ai;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kRowThreads / 64; ++w) {
            lse_merge(m, s, lm[w], ls[w]);
            if (lv[w] > av || (lv[w] == av && li[w] < ai)) {
                av = lv[w];
                ai = li[w];
            }
        }
        const size_t o = size_t(e) * p.nseg + sg;
        p.rs_m[o] = m;
        p.rs_s[o] = s;
        p.rs_v[o] = av;
        p.rs_i[o] = ai;
    }
}

// ------------------------------------------------------------------ accepted mass

struct AccMassParams {
    const float *U, *target;
    const void *W1, *W2;
    const float *temperature, *lse_q;
    int gamma, V, nbg, ntiles, tiles_per_chunk, nchunk, nseg;
    const int32_t *count, *ent_rho, *ent_trow, *ent_prev;
    const float *rs_m, *rs_s;
    float *mass;  // [entries, nchunk]
};

// A workgroup of 8 waves walks the tiles of one vocabulary chunk, one tile per
// stage, each wave holding 32 listed sampled rows.  Every stage is double
// buffered in LDS and loaded by direct loads one stage ahead: the tile's W2
// rows (shared by the workgroup) and, in wave-private regions, the rows'
// target and U_k entries.  The MFMA adds the bias tile onto the U_k tile; the
// two halves of a wave hold the two halves of the tile and add their sums
// once, at the end.
template <typename WT, int R, bool VEC>
__global__ __launch_bounds__(kAccThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void accept_mass_kernel(
    AccMassParams p) {
    using L = TileLDS<WT, R>;
    using TR = TileRows<VEC>;
    constexpr int NWV = kAccThreads / 64;
    __shared__ __attribute__((aligned(16))) uint8_t ldsW0[L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsW1[L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsU0[NWV * TR::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsU1[NWV * TR::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsT0[NWV * TR::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsT1[NWV * TR::BYTES];
    const int ns = p.count[0];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = lg / p.nbg, bg = lg % p.nbg;
    const int e0 = bg * NWV * 32;  // first list entry of the workgroup
    if (e0 >= ns) return;          // the whole workgroup is idle
    const int w0 = e0 + wave * 32;
    const bool wave_ok = w0 < ns;  // uniform across the wave
    const int n = lane & 31, h = lane >> 5;
    const int e = w0 + n;
    const bool ok = e < ns;
    const int ec = min(e, ns - 1);  // rows past the list repeat the last one; their sums are dropped
    const int rho = p.ent_rho[ec];
    const int trow_i = p.ent_trow[ec];
    const int prev = p.ent_prev[ec];
    const float sc = kLog2e / p.temperature[rho / p.gamma];
    const float lse2q = p.lse_q[rho] * kLog2e;
    float m = kNegInf, s = 0.f;
    for (int i = 0; i < p.nseg; ++i) lse_merge(m, s, p.rs_m[size_t(ec) * p.nseg + i], p.rs_s[size_t(ec) * p.nseg + i]);
    const float lse2t = m + fast_log2(s);

    const WT *W2 = static_cast<const WT *>(p.W2);
    EFrags<WT, R> ef;
    TileDMA<WT, R, kAccThreads> dma;
    dma.init(tid);
    TR su, stg;
    if (wave_ok) {
        ef.load(static_cast<const WT *>(p.W1) + size_t(prev) * R, h);
        stg.init(lane, p.target, size_t(p.V), [&](int r) { return __shfl(trow_i, r); });
        su.init(lane, p.U, size_t(p.V), [&](int r) { return __shfl(rho, r); });
    }
    const int roff = wave * TR::BYTES;

    const int t_begin = chunk * p.tiles_per_chunk;
    const int t_end = min(p.ntiles, t_begin + p.tiles_per_chunk);
    const bool tail = t_end * kTile > p.V;
    const int nfull = (t_end - t_begin) - (tail ? 1 : 0);
    float a0 = 0.f, a1 = 0.f;

    auto issue = [&](int t, uint8_t *w, uint8_t *ur, uint8_t *tr, auto clamp) __device__ {
        constexpr bool C = decltype(clamp)::value;
        dma.template issue<C>(W2, t * kTile, p.V, w, wave);
        if (wave_ok) {
            stg.template issue<C>(t * kTile, p.V, tr + roff, lane);
            su.template issue<C>(t * kTile, p.V, ur + roff, lane);
        }
    };
    auto stage = [&](int t, const uint8_t *w, const uint8_t *ur, const uint8_t *tr, bool masked) __device__ {
        f32x16_t pv = stg.read(tr + roff, lane);
        f32x16_t c = bias_tile_lds(ef, w, lane, su.read(ur + roff, lane));
        if (masked) {
            // value 4i+jj of lane (n, h) is entry 8i + 4h + jj of the tile
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (t * kTile + 8 * i + 4 * h + jj >= p.V) pv[4 * i + jj] = c[4 * i + jj] = kNegInf;
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            a0 += fminf(fast_exp2(__builtin_fmaf(pv[i], sc, -lse2t)), fast_exp2(__builtin_fmaf(c[i], sc, -lse2q)));
            a1 += fminf(fast_exp2(__builtin_fmaf(pv[i + 1], sc, -lse2t)),
                        fast_exp2(__builtin_fmaf(c[i + 1], sc, -lse2q)));
        }
    };

    using NoClamp = std::integral_constant<bool, false>;
    using Clamp = std::integral_constant<bool, true>;
    if (nfull > 0) issue(t_begin, ldsW0, ldsU0, ldsT0, NoClamp{});
    for (int i = 0; i < nfull; i += 2) {
        const int t = t_begin + i;
        __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of stage i have landed
        __syncthreads();                // ... and every thread's; the 1-buffers are free again
        if (i + 1 < nfull) issue(t + 1, ldsW1, ldsU1, ldsT1, NoClamp{});
        if (wave_ok) stage(t, ldsW0, ldsU0, ldsT0, false);
        if (i + 1 >= nfull) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // stage i + 1 has landed; the 0-buffers are free again
        if (i + 2 < nfull) issue(t + 2, ldsW0, ldsU0, ldsT0, NoClamp{});
        if (wave_ok) stage(t + 1, ldsW1, ldsU1, ldsT1, false);
    }
    if (tail) {
        __syncthreads();  // every wave is done with every buffer
        issue(t_end - 1, ldsW0, ldsU0, ldsT0, Clamp{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave_ok) stage(t_end - 1, ldsW0, ldsU0, ldsT0, true);
    }
    const float tot = half_sum(a0 + a1);
    if (h == 0 && ok) p.mass[size_t(e) * p.nchunk + chunk] = tot;
}

// ------------------------------------------------------------------ finish

struct AccFinishParams {
    const int32_t *count, *ent_rho, *x;
    int nchunk, nseg;
    const float *mass, *rs_v;
    const int32_t *rs_i;
    float *alpha_out;
};

__global__ __launch_bounds__(256) void accept_finish_kernel(AccFinishParams p) {
    const int ns = p.count[0], n = ns + p.count[1];
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const int rho = p.ent_rho[e];
    float alpha;
    if (e < ns) {
        const float *row = p.mass + size_t(e) * p.nchunk;
        float a[4] = {0.f, 0.f, 0.f, 0.f};
        int c = 0;
        for (; c + 4 <= p.nchunk; c += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] += row[c + u];
        }
        for (; c < p.nchunk; ++c) a[0] += row[c];
        alpha = (a[0] + a[1]) + (a[2] + a[3]);
    } else {
        float av = kNegInf;
        int ai = 0x7fffffff;
        for (int i = 0; i < p.nseg; ++i) {
            const float v2 = p.rs_v[size_t(e) * p.nseg + i];
            const int i2 = p.rs_i[size_t(e) * p.nseg + i];
            if (v2 > av || (v2 == av && i2 < ai)) {
                av = v2;
                ai = i2;
            }
        }
        if (ai == 0x7fffffff) ai = 0;  // every entry -inf: the first one is the argmax
        alpha = (ai == p.x[rho]) ? 1.f : 0.f;
    }
    p.alpha_out[rho] = alpha;
}

template <typename WT, int R>
hipError_t launch_accept_typed(const AcceptArgs &a, const AcceptPlan &pl, const AcceptWork &w, hipStream_t s) {
    hipError_t e;
    {
        AccPrepParams pp{a.ell, a.row_offsets, a.anchor, a.x, a.temperature, a.B, a.gamma, a.V, a.n_target_rows,
                         w.count, w.ent_rho, w.ent_trow, w.ent_prev, a.alpha_out, a.erow_mode};
        launch_kernel("accept_prep", accept_prep_kernel, dim3(1), dim3(1024), s, pp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool vec_t = reinterpret_cast<uintptr_t>(a.target) % 16 == 0 && a.V % 4 == 0;
    const bool vec_u = reinterpret_cast<uintptr_t>(a.U) % 16 == 0 && a.V % 4 == 0;
    {
        AccRowParams rp{a.target, a.temperature, a.gamma, a.V, pl.nseg, pl.seg_len,
                        w.count, w.ent_rho, w.ent_trow, w.rs_m, w.rs_s, w.rs_v, w.rs_i};
        const dim3 grid(unsigned(size_t(pl.maxent) * pl.nseg));
        if (vec_t)
            launch_kernel("accept_rowstats", accept_rowstats_kernel<true>, grid, dim3(kRowThreads), s, rp);
        else
            launch_kernel("accept_rowstats", accept_rowstats_kernel<false>, grid, dim3(kRowThreads), s, rp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        AccMassParams mp{};
        mp.U = a.U;
        mp.target = a.target;
        mp.W1 = a.W1;
        mp.W2 = a.W2;
        mp.temperature = a.temperature;
        mp.lse_q = a.lse_q;
        mp.gamma = a.gamma;
        mp.V = a.V;
        mp.nbg = pl.tile.nbg;
        mp.ntiles = pl.tile.ntiles;
        mp.tiles_per_chunk = pl.tile.tiles_per_chunk;
        mp.nchunk = pl.tile.nchunk;
        mp.nseg = pl.nseg;
        mp.count = w.count;
        mp.ent_rho = w.ent_rho;
        mp.ent_trow = w.ent_trow;
        mp.ent_prev = w.ent_prev;
        mp.rs_m = w.rs_m;
        mp.rs_s = w.rs_s;
        mp.mass = w.mass;
        if (vec_u && vec_t)
            launch_kernel("accept_mass", (accept_mass_kernel<WT, R, true>), dim3(pl.tile.blocks), dim3(kAccThreads), s, mp);
        else
            launch_kernel("accept_mass", (accept_mass_kernel<WT, R, false>), dim3(pl.tile.blocks), dim3(kAccThreads), s, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        AccFinishParams fp{w.count, w.ent_rho, a.x, pl.tile.nchunk, pl.nseg, w.mass, w.rs_v, w.rs_i, a.alpha_out};
        launch_kernel("accept_finish", accept_finish_kernel, dim3((pl.maxent + 255) / 256), dim3(256), s, fp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

AcceptPlan accept_plan(int B, int gamma, int V) {
    AcceptPlan p{};
    p.maxent = B * gamma;
    // row statistics: about 2048 workgroups when every row is listed, in
    // segments of whole float4 groups
    const int n4 = (V + 3) / 4;
    const int want = std::min(16, std::max(1, (2048 + p.maxent - 1) / p.maxent));
    p.seg_len = 4 * ((n4 + want - 1) / want);
    p.nseg = (V + p.seg_len - 1) / p.seg_len;
    // accepted mass: 8-wave workgroups of 256 listed rows, one a CU (the
    // stages take 160 KB of LDS at bf16 rank 256), about 256 of them
    p.tile = tile_walk_plan(p.maxent, V, kAccThreads / 64, 256, 1);
    return p;
}

AcceptWork accept_carve(void *ws, int B, int gamma, const AcceptPlan &p, size_t *bytes) {
    (void)B;
    (void)gamma;
    Carve c(ws);
    AcceptWork w{};
    w.count = c.take<int32_t>(4);
    w.ent_rho = c.take<int32_t>(p.maxent);
    w.ent_trow = c.take<int32_t>(p.maxent);
    w.ent_prev = c.take<int32_t>(p.maxent);
    const size_t nr = size_t(p.maxent) * p.nseg;
    w.rs_m = c.take<float>(nr);
    w.rs_s = c.take<float>(nr);
    w.rs_v = c.take<float>(nr);
    w.rs_i = c.take<int32_t>(nr);
    w.mass = c.take<float>(size_t(p.maxent) * p.tile.nchunk);
    if (bytes) *bytes = c.off + 256;
    return w;
}

hipError_t launch_accept(const AcceptArgs &a, const AcceptPlan &p, const AcceptWork &w, hipStream_t s) {
    if (a.wdtype == 0) {
        switch (a.r) {
            case 16: return launch_accept_typed<uint16_t, 16>(a, p, w, s);
            case 32: return launch_accept_typed<uint16_t, 32>(a, p, w, s);
            case 64: return launch_accept_typed<uint16_t, 64>(a, p, w, s);
            case 128: return launch_accept_typed<uint16_t, 128>(a, p, w, s);
            case 256: return launch_accept_typed<uint16_t, 256>(a, p, w, s);
        }
    } else {
        switch (a.r) {
            case 16: return launch_accept_typed<float, 16>(a, p, w, s);
            case 32: return launch_accept_typed<float, 32>(a, p, w, s);
            case 64: return launch_accept_typed<float, 64>(a, p, w, s);
            case 128: return launch_accept_typed<float, 128>(a, p, w, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dspark
