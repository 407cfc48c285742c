// draft.hip -- the draft half of a DSpark round on gfx950: the sequential
// Markov-head sampling loop over block positions k = 1..gamma.
//
// Method (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
// section 3.2 Sequential Stage; "DeepSeek DSpark explained"
// (share.concentrate1.com), section 03): with x_0 the anchor,
//   B_k = W1[x_{k-1}] W2^T,   q_k = softmax((U_k + B_k) / T),   x_k ~ q_k,
// one position after another, each step reading the token the previous one
// sampled.  The draw is Gumbel-max with Philox noise; T = 0 is greedy.
//
// Per position k the work is one pass over the [B, V] plane:
//   draft_step    one wave per (32 requests x vocabulary chunk): the bias
//                 tile on MFMA (bf16 32x32x16, or f32 32x32x2), + U_k, the
//                 temperature, an online max / sum of exp2 (base-2 softmax
//                 statistics) and the Gumbel-perturbed best score, all in
//                 registers; per (request, chunk) partials go to the workspace.
//   draft_reduce  one wave per request: merges the chunk partials into x_k,
//                 lse_k, q_k(x_k) and the top-two gap.
// The bias plane is never stored; HBM traffic per step is U_k, W2 and the
// gathered W1 rows.
#include "device_common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace dspark {

namespace {

struct StepParams {
    const float *U;  // U + (k - 1) * V: row b at U + b * u_stride
    size_t u_stride;
    const void *W1, *W2;
    const int32_t *xprev;  // x_{k-1} of request b at xprev[b * xprev_stride]
    int xprev_stride;
    const float *temperature;
    int B, V, k;
    uint32_t key0, key1, round32;
    int nbb, tiles_per_chunk, nchunk, total_waves;
    int vec;  // U rows allow aligned 16-byte loads
    float *pm, *ps, *pb, *p2;
    int32_t *pi;
};

template <typename WT, int R, bool TRACK2>
__global__ __launch_bounds__(256) void draft_step_kernel(StepParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    if (gw >= p.total_waves) return;
    const int bb = gw % p.nbb;
    const int chunk = gw / p.nbb;
    const int n = lane & 31, h = lane >> 5;
    const int b = bb * 32 + n;
    const bool row_ok = b < p.B;
    const int bc = row_ok ? b : p.B - 1;

    int prev = p.xprev[size_t(bc) * p.xprev_stride];
    prev = min(max(prev, 0), p.V - 1);
    const float T = p.temperature[bc];
    const bool sampled = T > 0.f;
    const float sc = sampled ? kLog2e / T : 1.0f;  // base-2 logits; greedy keeps raw logits
    const float gm = sampled ? 1.0f : 0.0f;        // greedy rows ignore the noise

    const WT *W1 = static_cast<const WT *>(p.W1);
    const WT *W2 = static_cast<const WT *>(p.W2);
    EFrags<WT, R> ef;
    ef.load(W1 + size_t(prev) * R, h);
    const float *urow = p.U + size_t(bc) * p.u_stride;
    const bool vec = p.vec != 0;

    const int v_begin = chunk * p.tiles_per_chunk * 32;
    const int v_end = min(p.V, v_begin + p.tiles_per_chunk * 32);
    float m_run = kNegInf, s_run = 0.f;
    float best = kNegInf, second = kNegInf;
    int bidx = v_begin + 4 * h;  // lowest entry of this lane: wins if everything is -inf

    for (int v0 = v_begin; v0 < v_end; v0 += 32) {
        const int vrow = min(v0 + n, p.V - 1);
        const f32x16_t acc = bias_tile(ef, W2 + size_t(vrow) * R, h);
        float z[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 u = load4_masked(urow, v0 + 8 * i + 4 * h, p.V, vec);
#pragma unroll
            for (int j = 0; j < 4; ++j) z[4 * i + j] = (f4get(u, j) + acc[4 * i + j]) * sc;
        }
        float mt = z[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mt = fmaxf(mt, z[e]);
        const float mn = fmaxf(m_run, mt);
        const float ms = (mn == kNegInf) ? 0.f : mn;
        float add = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) add += fast_exp2(z[e] - ms);
        s_run = s_run * fast_exp2(m_run - ms) + add;
        m_run = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = draft_noise_block(p.k, uint32_t(v0 >> 2) + uint32_t(2 * i + h), uint32_t(b),
                                              p.round32, p.key0, p.key1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float score = __builtin_fmaf(gumbel2(u4get(w, j)), gm, z[4 * i + j]);
                if (TRACK2) second = fmaxf(second, fminf(score, best));
                if (score > best) {
                    best = score;
                    bidx = v0 + 8 * i + 4 * h + j;
                }
            }
        }
    }
    // merge the two lane halves that share a request
    {
        const float m2 = __shfl_xor(m_run, 32), s2 = __shfl_xor(s_run, 32);
        const float b2 = __shfl_xor(best, 32), c2 = __shfl_xor(second, 32);
        const int i2 = __shfl_xor(bidx, 32);
        lse_merge(m_run, s_run, m2, s2);
        best_merge(best, bidx, second, b2, i2, c2);
    }
    if (h == 0 && row_ok) {
        const size_t o = size_t(b) * p.nchunk + chunk;
        p.pm[o] = m_run;
        p.ps[o] = s_run;
        p.pb[o] = best;
        p.pi[o] = bidx;
        if (TRACK2) p.p2[o] = second;
    }
}

struct ReduceParams {
    const float *U;  // U + (k - 1) * V
    size_t u_stride;
    const void *W1, *W2;
    const int32_t *xprev;
    int xprev_stride;
    const float *temperature;
    int B, V, k, gamma, nchunk;
    const float *pm, *ps, *pb, *p2;
    const int32_t *pi;
    int32_t *x_out;
    float *lse_out, *qx_out, *margin_out;
};

template <typename WT, int R>
__global__ __launch_bounds__(256) void draft_reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= p.B) return;
    const bool track2 = p.margin_out != nullptr;
    float m = kNegInf, s = 0.f, best = kNegInf, second = kNegInf;
    int idx = 0x7fffffff;
    for (int c = lane; c < p.nchunk; c += 64) {
        const size_t o = size_t(b) * p.nchunk + c;
        lse_merge(m, s, p.pm[o], p.ps[o]);
        best_merge(best, idx, second, p.pb[o], p.pi[o], track2 ? p.p2[o] : kNegInf);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
        const float b2 = __shfl_xor(best, off), c2 = __shfl_xor(second, off);
        const int i2 = __shfl_xor(idx, off);
        lse_merge(m, s, m2, s2);
        best_merge(best, idx, second, b2, i2, c2);
    }
    const int x = min(max(idx, 0), p.V - 1);
    int prev = p.xprev[size_t(b) * p.xprev_stride];
    prev = min(max(prev, 0), p.V - 1);
    // z(x_k): recompute the one bias entry the sample landed on
    const WT *W1 = static_cast<const WT *>(p.W1);
    const WT *W2 = static_cast<const WT *>(p.W2);
    float d = 0.f;
    for (int i = lane; i < R; i += 64) {
        float a, w;
        if constexpr (sizeof(WT) == 2) {
            a = __uint_as_float(uint32_t(W1[size_t(prev) * R + i]) << 16);
            w = __uint_as_float(uint32_t(W2[size_t(x) * R + i]) << 16);
        } else {
            a = W1[size_t(prev) * R + i];
            w = W2[size_t(x) * R + i];
        }
        d = __builtin_fmaf(a, w, d);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
    if (lane == 0) {
        const float T = p.temperature[b];
        const size_t o = size_t(b) * p.gamma + (p.k - 1);
        p.x_out[o] = x;
        if (T > 0.f) {
            const float sc = kLog2e / T;
            const float z2x = (p.U[size_t(b) * p.u_stride + x] + d) * sc;
            const float lse2 = m + fast_log2(s);
            p.lse_out[o] = lse2 * kLn2;
            p.qx_out[o] = fast_exp2(z2x - lse2);
            if (track2) p.margin_out[o] = (best - second) * kLn2;
        } else {
            p.lse_out[o] = m;
            p.qx_out[o] = 1.0f;
            if (track2) p.margin_out[o] = best - second;
        }
    }
}

template <typename WT, int R>
hipError_t launch_typed(const DraftArgs &a, const DraftPlan &pl, const DraftWork &w, hipStream_t s) {
    const bool track2 = a.margin_out != nullptr;
    const bool vec = (reinterpret_cast<uintptr_t>(a.U) % 16 == 0) && (a.V % 4 == 0);
    for (int k = 1; k <= a.gamma; ++k) {
        StepParams sp{};
        sp.U = a.U + size_t(k - 1) * a.V;
        sp.u_stride = size_t(a.gamma) * a.V;
        sp.W1 = a.W1;
        sp.W2 = a.W2;
        sp.xprev = (k == 1) ? a.anchor : a.x_out + (k - 2);
        sp.xprev_stride = (k == 1) ? 1 : a.gamma;
        sp.temperature = a.temperature;
        sp.B = a.B;
        sp.V = a.V;
        sp.k = k;
        sp.key0 = a.key0;
        sp.key1 = a.key1;
        sp.round32 = a.round32;
        sp.nbb = pl.nbb;
        sp.tiles_per_chunk = pl.tiles_per_chunk;
        sp.nchunk = pl.nchunk;
        sp.total_waves = pl.total_waves;
        sp.vec = vec;
        sp.pm = w.pm;
        sp.ps = w.ps;
        sp.pb = w.pb;
        sp.p2 = w.p2;
        sp.pi = w.pi;
        int t = prof_begin("draft_step", s);
        if (track2)
            hipLaunchKernelGGL((draft_step_kernel<WT, R, true>), dim3(pl.blocks), dim3(256), 0, s, sp);
        else
            hipLaunchKernelGGL((draft_step_kernel<WT, R, false>), dim3(pl.blocks), dim3(256), 0, s, sp);
        prof_end(t, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;

        ReduceParams rp{};
        rp.U = sp.U;
        rp.u_stride = sp.u_stride;
        rp.W1 = a.W1;
        rp.W2 = a.W2;
        rp.xprev = sp.xprev;
        rp.xprev_stride = sp.xprev_stride;
        rp.temperature = a.temperature;
        rp.B = a.B;
        rp.V = a.V;
        rp.k = k;
        rp.gamma = a.gamma;
        rp.nchunk = pl.nchunk;
        rp.pm = w.pm;
        rp.ps = w.ps;
        rp.pb = w.pb;
        rp.p2 = w.p2;
        rp.pi = w.pi;
        rp.x_out = a.x_out;
        rp.lse_out = a.lse_out;
        rp.qx_out = a.qx_out;
        rp.margin_out = a.margin_out;
        t = prof_begin("draft_reduce", s);
        hipLaunchKernelGGL((draft_reduce_kernel<WT, R>), dim3((a.B + 3) / 4), dim3(256), 0, s, rp);
        prof_end(t, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

DraftPlan draft_plan(int B, int V) {
    DraftPlan p{};
    p.nbb = (B + 31) / 32;
    p.ntiles = (V + 31) / 32;
    // aim for ~4096 waves (16 per CU) so every SIMD keeps several waves
    const long long work = 1LL * p.nbb * p.ntiles;
    const long long target = 4096;
    p.tiles_per_chunk = int(std::max<long long>(1, (work + target - 1) / target));
    p.nchunk = (p.ntiles + p.tiles_per_chunk - 1) / p.tiles_per_chunk;
    p.total_waves = p.nbb * p.nchunk;
    p.blocks = (p.total_waves + 3) / 4;
    return p;
}

DraftWork draft_carve(void *ws, int B, const DraftPlan &p, size_t *bytes) {
    Carve c(ws);
    const size_t n = size_t(B) * p.nchunk;
    DraftWork w{};
    w.pm = c.take<float>(n);
    w.ps = c.take<float>(n);
    w.pb = c.take<float>(n);
    w.p2 = c.take<float>(n);
    w.pi = c.take<int32_t>(n);
    if (bytes) *bytes = c.off + 256;
    return w;
}

hipError_t launch_draft(const DraftArgs &a, const DraftPlan &p, const DraftWork &w, hipStream_t s) {
    if (a.wdtype == 0) {
        switch (a.r) {
            case 16: return launch_typed<uint16_t, 16>(a, p, w, s);
            case 32: return launch_typed<uint16_t, 32>(a, p, w, s);
            case 64: return launch_typed<uint16_t, 64>(a, p, w, s);
            case 128: return launch_typed<uint16_t, 128>(a, p, w, s);
            case 256: return launch_typed<uint16_t, 256>(a, p, w, s);
        }
    } else {
        switch (a.r) {
            case 16: return launch_typed<float, 16>(a, p, w, s);
            case 32: return launch_typed<float, 32>(a, p, w, s);
            case 64: return launch_typed<float, 64>(a, p, w, s);
            case 128: return launch_typed<float, 128>(a, p, w, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dspark
