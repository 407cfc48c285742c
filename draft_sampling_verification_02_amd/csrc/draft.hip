// draft.hip -- the draft half of a DSpark round on gfx950: the sequential
// Markov-head sampling loop over block positions k = 1..gamma.
//
// Method (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
// section 3.2 Sequential Stage; "DeepSeek DSpark explained"
// (share.concentrate1.com), section 03): with x_0 the anchor,
//   B_k = W1[x_{k-1}] W2^T,   q_k = softmax((U_k + B_k) / T),   x_k ~ q_k,
// one position after another, each step reading the token the previous one
// sampled.  T = 0 is greedy.  The draw is a two-level Gumbel-max: a Gumbel
// race over the logsumexp of 32-entry vocabulary tiles (Philox stream 3),
// then one over the entries of the winning tile (stream 0) -- an exact draw
// from q_k that needs per-entry noise for a single tile only.
//
// Per position k the work is one pass over the [B, V] plane:
//   draft_step    a workgroup of up to 8 waves (32 requests each) walks the
//                 vocabulary tiles of one chunk, two tiles a stage: the
//                 stage's W2 rows (shared by the waves) and each wave's U_k
//                 entries are staged in LDS by direct loads, double buffered.
//                 The U_k entries seed the MFMA accumulators (bf16 32x32x16,
//                 or f32 32x32x2), which add the bias tile; 1/T gives the
//                 tile's base-2 logsumexp, which feeds both the running
//                 softmax sum and the tile race.
//   draft_reduce  one wave per request: merges the chunk partials (row
//                 logsumexp, best tile), recomputes the winning tile's 32
//                 logits on the vector ALUs and races their entry noise:
//                 x_k, lse_k, q_k(x_k) and the draw's margin.  For the next
//                 position it also writes W1[x_k] as a packed fragment block
//                 (it fetches the W1 rows of the whole winning tile with the
//                 tile's W2 rows, so the chosen row needs no further trip).
// The bias plane is never stored; HBM traffic per step is U_k, W2 and the
// gathered W1 rows.
#include "device_common.hpp"
#include "internal.hpp"
#include "stage.hpp"

#include <algorithm>
#include <type_traits>

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
    int erows;  // rows of W1 (the E rows are W1 + xprev * R, clamped below erows)
    uint32_t key0, key1, round32;
    int nbb, nw, nbg, ntiles, tiles_per_chunk, nchunk;
    int vec;  // U rows allow aligned 16-byte loads
    float *pm, *ps, *pb, *p2;
    int32_t *pi;
    const uint4 *ep;  // PACKED instances: the E rows of every request as PackedE blocks
};

// s_waitcnt immediate that waits for all but the n most recent vector memory
// operations of this wave (lgkm and exp counts left free)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

constexpr int kStepThreads = 512;  // 8 waves: one 32-request block each

// One workgroup of 8 waves walks the tiles [t_begin, t_end) of one vocabulary
// chunk, two tiles per stage: the pair's 64 W2 rows are staged in LDS by
// direct loads (two named buffers, so that the wait for one stage never waits
// for the next) and so are the pair's U_k entries (one region per wave,
// refilled as soon as the wave has read it); the U_k entries seed the MFMA
// accumulators, and after the two MFMA chains a lane-half swap hands the
// first tile of the pair to lanes 0..31 and the second to lanes 32..63.  A
// last stage that runs past the vocabulary is done on its own, after the loop.
// PACKED: the E rows come as PackedE blocks, written by the previous
// position's reduce, so that the fragments go out first, as whole 1 KiB loads
// with no dependency; otherwise every wave gathers its 32 rows of W1 (or of
// the head's rows) from x_{k-1}.
template <typename WT, int R, bool TRACK2, bool VEC, bool PACKED>
__global__ __launch_bounds__(kStepThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void draft_step_kernel(StepParams p) {
    using L = TileLDS<WT, R>;
    using SU = StageRows<VEC>;
    __shared__ __attribute__((aligned(16))) uint8_t ldsA[2 * L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsB[2 * L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsU[(kStepThreads / 64) * SU::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = lg / p.nbg, bg = lg % p.nbg;
    const int bb = bg * (kStepThreads / 64) + wave;
    const bool wave_ok = bb < p.nbb;  // uniform across the wave
    const int n = lane & 31, h = lane >> 5;
    const int b = bb * 32 + n;
    const bool row_ok = wave_ok && b < p.B;
    const int bc = min(b, p.B - 1);

    const WT *W2 = static_cast<const WT *>(p.W2);
    StageDMA<WT, R, kStepThreads> dma;
    dma.init(tid);
    SU su;  // every wave (rows past the batch repeat its last request)
    su.init(lane, p.U, p.u_stride, [&](int r) { return min(bb * 32 + r, p.B - 1); });
    uint8_t *uregion = ldsU + wave * SU::BYTES;
    const int t_begin = chunk * p.tiles_per_chunk;
    const int t_end = min(p.ntiles, t_begin + p.tiles_per_chunk);
    const int nst = (t_end - t_begin + 1) >> 1;  // stages of two tiles
    const bool tail = (t_begin + 2 * nst) * kTile > p.V;
    const int nfull = nst - (tail ? 1 : 0);
    auto v0_of = [&](int i) { return (t_begin + 2 * i) * kTile; };

    // x_{k-1} first, then the first stage's loads, which need nothing but the
    // tile walk, then the W1 gather: the stage streams in while the x_{k-1}
    // round trip and the gather resolve (loads retire in order, so waiting
    // for x_{k-1} leaves the stage in flight).  The stage is issued by every
    // wave and clamped to the vocabulary, so that the number of loads in
    // flight is the same on every path; a chunk that is only a tail stage
    // reloads the buffers after a full barrier.
    // The compiler does not count direct-to-LDS loads as younger than a
    // register load and would drain the stage before the gather, so x_{k-1}
    // and T are loaded and waited for in asm: with no more than this wave's
    // own stage loads in flight (at least NI + MIN_PER_WAVE of them, issued
    // after), both have landed.
    float T;
    EFrags<WT, R> ef;
    if constexpr (PACKED) {
        // the fragments and T first, then the first stage: nothing here waits
        // for anything before the first stage has landed (the padded rows of
        // the last block hold stale fragments; their columns are never written)
        T = p.temperature[bc];
        if (wave_ok) ef.load_packed(p.ep + size_t(bb) * PackedE<WT, R>::BLOCK, lane);
        __builtin_amdgcn_sched_barrier(0);
        dma.template issue<true>(W2, v0_of(0), p.V, ldsA, wave);
        su.template issue<true>(v0_of(0), p.V, uregion, lane);
    } else {
        int prev;
        asm volatile("global_load_dword %0, %1, off" : "=v"(prev) : "v"(p.xprev + size_t(bc) * p.xprev_stride) : "memory");
        asm volatile("global_load_dword %0, %1, off" : "=v"(T) : "v"(p.temperature + bc) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        dma.template issue<true>(W2, v0_of(0), p.V, ldsA, wave);
        su.template issue<true>(v0_of(0), p.V, uregion, lane);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(%2)" : "+v"(prev), "+v"(T) : "n"(SU::NI + decltype(dma)::MIN_PER_WAVE));
        prev = min(max(prev, 0), p.erows - 1);
        if (wave_ok) ef.load(static_cast<const WT *>(p.W1) + size_t(prev) * R, h);
    }
    const bool sampled = T > 0.f;
    const float sc = sampled ? kLog2e / T : 1.0f;  // base-2 logits; greedy keeps raw logits
    TileRace st{kNegInf, 0.f, kNegInf, kNegInf, t_begin};
    uint4 tw = make_uint4(0u, 0u, 0u, 0u);

    // stage at tile t0 (even): U_k from the wave's region, W2 from buf; next_v0
    // >= 0 refills the region with the next stage's U_k once it has been read
    auto stage = [&](const uint8_t *buf, int t0, int next_v0, bool masked) __device__ {
        f32x16_t c0, c1;
        su.read(uregion, lane, c0, c1);
        if (next_v0 >= 0) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the region has been read
            su.template issue<false>(next_v0, p.V, uregion, lane);
        }
        bias_pair_lds(ef, buf, lane, c0, c1);
        swap_halves(c0, c1);
        if (masked) {
            const int vb = (t0 + h) * kTile;  // this lane's tile: c0 rows 8i+j, c1 rows 8i+4+j
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (vb + 8 * i + j >= p.V) c0[4 * i + j] = kNegInf;
                    if (vb + 8 * i + 4 + j >= p.V) c1[4 * i + j] = kNegInf;
                }
        }
        // t0 is even, so both tiles of the pair share one noise block; tile
        // t0 + h takes word (t0 & 3) + h
        if (t0 == t_begin || (t0 & 3) == 0)
            tw = noise_block(kStreamDraftTile, p.k, uint32_t(t0) >> 2, uint32_t(b), p.round32, p.key0, p.key1);
        const uint32_t w_lo = (t0 & 2) ? tw.z : tw.x, w_hi = (t0 & 2) ? tw.w : tw.y;
        race_tile<TRACK2>(st, c0, c1, sc, sampled, t0 + h, gumbel2(h ? w_hi : w_lo));
    };

    for (int i = 0; i < nfull; i += 2) {
        __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of stage i have landed
        __syncthreads();                // ... and every thread's; ldsB is free again
        if (i + 1 < nfull) dma.template issue<false>(W2, v0_of(i + 1), p.V, ldsB, wave);
        if (wave_ok) stage(ldsA, t_begin + 2 * i, i + 1 < nfull ? v0_of(i + 1) : -1, false);
        if (i + 1 >= nfull) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // stage i + 1 has landed; ldsA is free again
        if (i + 2 < nfull) dma.template issue<false>(W2, v0_of(i + 2), p.V, ldsA, wave);
        if (wave_ok) stage(ldsB, t_begin + 2 * (i + 1), i + 2 < nfull ? v0_of(i + 2) : -1, false);
    }
    if (tail) {
        __syncthreads();  // every wave is done with both W2 buffers and its region
        dma.template issue<true>(W2, v0_of(nfull), p.V, ldsA, wave);
        if (wave_ok) su.template issue<true>(v0_of(nfull), p.V, uregion, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave_ok) stage(ldsA, t_begin + 2 * nfull, -1, true);
    }
    // the two lane halves raced alternate tiles of the same request
    {
        const float m2 = bfly<5>(st.m), s2 = bfly<5>(st.s);
        const float b2 = bfly<5>(st.best), c2 = bfly<5>(st.second);
        const int i2 = bfly<5>(st.bt);
        lse_merge(st.m, st.s, m2, s2);
        best_merge(st.best, st.bt, st.second, b2, i2, TRACK2 ? c2 : kNegInf);
    }
    if (h == 0 && row_ok) {
        const size_t o = size_t(b) * p.nchunk + chunk;
        p.pm[o] = st.m;
        p.ps[o] = st.s;
        p.pb[o] = st.best;
        p.pi[o] = st.bt;
        if (TRACK2) p.p2[o] = st.second;
    }
}

struct ReduceParams {
    const float *U;  // U + (k - 1) * V
    size_t u_stride;
    const void *W1, *W2;
    const int32_t *xprev;
    int xprev_stride;
    const float *temperature;
    int B, V, k, gamma, nchunk, ntiles;
    int erows;  // as for StepParams
    uint32_t key0, key1, round32;
    const float *pm, *ps, *pb, *p2;
    const int32_t *pi;
    int32_t *x_out;
    float *lse_out, *qx_out, *margin_out;
    // confidence head (used by the CONF instances only)
    const float *hidden;  // h_k of request b at hidden + b * h_stride
    size_t h_stride;
    const float *conf_w;  // [d + r]: the h_k part, then the W1[x_{k-1}] part
    int d, hvec;          // hvec: h rows and conf_w allow aligned 16-byte loads
    const float *conf_tau;  // [gamma] temperatures of the head's logit, or nullptr (1)
    float *conf_out, *surv_out;
    uint4 *ep_out;  // PackedE blocks of W1[x_k] for the next position's step, or nullptr
};

// w_h . h_k, this lane's share (the wave sums it): lane l takes entries
// l, l + 64, ... (as float4 pieces when hvec); every load is issued before
// the first product for d up to 1024 (float4) or 512 (float).
__device__ __forceinline__ float conf_hidden_part(const ReduceParams &p, int b, int lane) {
    const float *hk = p.hidden + size_t(b) * p.h_stride;
    float acc = 0.f;
    if (p.hvec) {
        const int n4 = p.d >> 2;
        const float4 *h4 = reinterpret_cast<const float4 *>(hk);
        const float4 *w4 = reinterpret_cast<const float4 *>(p.conf_w);
        for (int i0 = 0; i0 < n4; i0 += 64 * 4) {
            float4 hv[4], wv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = min(i0 + lane + 64 * u, n4 - 1);  // clamped, masked below
                hv[u] = h4[i];
                wv[u] = w4[i];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float t = hv[u].x * wv[u].x;
                t = __builtin_fmaf(hv[u].y, wv[u].y, t);
                t = __builtin_fmaf(hv[u].z, wv[u].z, t);
                t = __builtin_fmaf(hv[u].w, wv[u].w, t);
                acc += (i0 + lane + 64 * u < n4) ? t : 0.f;
            }
        }
    } else {
        for (int i0 = 0; i0 < p.d; i0 += 64 * 8) {
            float hv[8], wv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(i0 + lane + 64 * u, p.d - 1);
                hv[u] = hk[i];
                wv[u] = p.conf_w[i];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += (i0 + lane + 64 * u < p.d) ? hv[u] * wv[u] : 0.f;
        }
    }
    return acc;
}

// One wave per request.  The loads that do not depend on the winning tile
// (the W1 row, the chunk partials) go out together; the winning tile's W2
// rows and U entries go out together once it is known.
// CONF instances also evaluate the confidence head of position k,
//   c_k = sigmoid(w . [h_k, W1[x_{k-1}]])  (bias-free linear layer),
// and the prefix survival a_k = a_{k-1} c_k (a_{k-1} written by the previous
// position's launch): the gathered W1 row is already at hand here, and the
// h_k row streams in beside the partials.
// One wave a workgroup, so that the requests' tile fetches (their W2 and W1
// rows, 32 KiB a request) spread over every CU.
constexpr int kReduceWaves = 1;

template <typename WT, int R, bool CONF>
__global__ __launch_bounds__(64 * kReduceWaves) void draft_reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kReduceWaves + (threadIdx.x >> 6);
    if (b >= p.B) return;
    const bool track2 = p.margin_out != nullptr;
    // level 1: row logsumexp and the winning tile, four chunks a lane per
    // batch.  The loads go out first and unconditionally (an index past the
    // chunks re-reads chunk 0 and is masked after), so that the first batch
    // is in flight while x_{k-1} and its W1 row are fetched.
    constexpr int PC = 4;
    float cm[PC], cs[PC], cb[PC], c2[PC];
    int ci[PC];
    auto load_batch = [&](int c0) __device__ {
#pragma unroll
        for (int u = 0; u < PC; ++u) {
            const int c = c0 + lane + 64 * u;
            const size_t o = size_t(b) * p.nchunk + (c < p.nchunk ? c : 0);
            cm[u] = p.pm[o];
            cs[u] = p.ps[o];
            cb[u] = p.pb[o];
            ci[u] = p.pi[o];
            c2[u] = p.p2[o];  // written only when the margin is tracked; masked below otherwise
        }
    };
    load_batch(0);
    __builtin_amdgcn_sched_barrier(0);  // keep the batch ahead of the dependent W1 fetch
    int prev = p.xprev[size_t(b) * p.xprev_stride];
    const float T = p.temperature[b];
    float conf_s = 0.f, a_prev = 1.f, conf_t = 1.f;
    if constexpr (CONF) {
        if (p.k > 1) a_prev = p.surv_out[size_t(b) * p.gamma + p.k - 2];
        if (p.conf_tau) conf_t = p.conf_tau[p.k - 1];
        if (p.d > 0) conf_s = conf_hidden_part(p, b, lane);
    }
    prev = min(max(prev, 0), p.erows - 1);
    using TD = TileDot<WT, R>;
    // the chunk of W1[x_{k-1}] this lane dots with the winning tile's rows
    const uint4 ech = reinterpret_cast<const uint4 *>(static_cast<const WT *>(p.W1) + size_t(prev) * R)[lane % TD::CPR];
    if constexpr (CONF) {
        // w_e . W1[x_{k-1}], entries lane, lane + 64, ...
        const WT *e = static_cast<const WT *>(p.W1) + size_t(prev) * R;
#pragma unroll
        for (int i = lane; i < R; i += 64) {
            float ev;
            if constexpr (sizeof(WT) == 2)
                ev = __uint_as_float(uint32_t(e[i]) << 16);
            else
                ev = e[i];
            conf_s = __builtin_fmaf(p.conf_w[p.d + i], ev, conf_s);
        }
    }
    float m = kNegInf, s = 0.f, best = kNegInf, second = kNegInf;
    int bt = 0x7fffffff;
    for (int c0 = 0; c0 < p.nchunk; c0 += 64 * PC) {
        if (c0 > 0) load_batch(c0);
#pragma unroll
        for (int u = 0; u < PC; ++u) {
            if (c0 + lane + 64 * u < p.nchunk) {
                lse_merge(m, s, cm[u], cs[u]);
                best_merge(best, bt, second, cb[u], ci[u], track2 ? c2[u] : kNegInf);
            }
        }
    }
    bfly_steps<0, 6>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float m2 = bfly<S>(m), s2 = bfly<S>(s), b2 = bfly<S>(best), c2 = bfly<S>(second);
        const int i2 = bfly<S>(bt);
        lse_merge(m, s, m2, s2);
        best_merge(best, bt, second, b2, i2, c2);
    });
    const int tile = min(max(bt, 0), p.ntiles - 1);
    // level 2: the winning tile's logits on the vector ALUs, then the entry race
    const bool sampled = T > 0.f;
    const float sc = sampled ? kLog2e / T : 1.0f;
    // this lane's entry of the tile (lanes l and l ^ 1 share one)
    const int v = tile * kTile + TD::row_of(lane);
    const bool valid = v < p.V;
    const int vc = min(v, p.V - 1);
    // the tile's W2 rows and, for the next position's packed block, the W1
    // rows of every candidate, all in whole lines
    TD w2t, w1t;
    w2t.load(static_cast<const WT *>(p.W2), tile * kTile, p.V - 1, lane);
    if (p.ep_out) w1t.load(static_cast<const WT *>(p.W1), tile * kTile, p.V - 1, lane);
    const float u_v = p.U[size_t(b) * p.u_stride + vc];
    const float d = w2t.dot(ech);
    const float logit = valid ? u_v + d : kNegInf;
    const float z2 = logit * sc;
    float score = logit;
    if (sampled) score = z2 + gumbel2(noise_word(kStreamDraft, p.k, uint32_t(vc), uint32_t(b), p.round32, p.key0, p.key1));
    if (lane & 1) score = kNegInf;  // the odd lanes duplicate the even ones
    float s1 = score, s2 = kNegInf;
    int xi = v;
    bfly_steps<0, 6>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float b2 = bfly<S>(s1), c2 = bfly<S>(s2);
        const int i2 = bfly<S>(xi);
        best_merge(s1, xi, s2, b2, i2, c2);
    });
    const int x = min(max(xi, tile * kTile), p.V - 1);
    const int wn = x - tile * kTile;  // the winner's row in the tile
    const float z2x = __shfl(z2, TD::lane_of(wn));
    if (p.ep_out) {
        // W1[x]'s chunks sit in load slot wn / RPI of the lanes of row group wn % RPI
        const int js = wn / TD::RPI;  // uniform
        uint4 row = w1t.w[0];
#pragma unroll
        for (int j = 1; j < TD::NI; ++j)
            if (j == js) row = w1t.w[j];
        if (lane / TD::CPR == wn % TD::RPI)
            p.ep_out[size_t(b >> 5) * PackedE<WT, R>::BLOCK + PackedE<WT, R>::slot(b & 31, lane % TD::CPR)] = row;
    }
    if constexpr (CONF) bfly_steps<0, 6>([&](auto st) { conf_s += bfly<decltype(st)::value>(conf_s); });
    if (lane == 0) {
        const size_t o = size_t(b) * p.gamma + (p.k - 1);
        p.x_out[o] = x;
        if constexpr (CONF) {
            const float c = 1.0f / (1.0f + __expf(-conf_s / conf_t));
            p.conf_out[o] = c;
            p.surv_out[o] = a_prev * c;
        }
        const float gap = fminf(best - second, s1 - s2);
        if (sampled) {
            const float lse2 = m + fast_log2(s);
            p.lse_out[o] = lse2 * kLn2;
            p.qx_out[o] = fast_exp2(z2x - lse2);
            if (track2) p.margin_out[o] = gap * kLn2;
        } else {
            p.lse_out[o] = m;
            p.qx_out[o] = 1.0f;
            if (track2) p.margin_out[o] = gap;
        }
    }
}

// ---- the bias product alone (a diagnostic of the matrix-unit tiling)

struct GemmParams {
    const uint4 *ep;  // PackedE blocks of the rows W1[idx[b]]
    const void *W2;
    int B, V;
    int nbb, nbg, ntiles, tiles_per_chunk, nchunk;
    float *pm;  // [B, nchunk] per-chunk row maxima
};

// The gather W1[idx[b]] into PackedE blocks: one thread per 16-byte chunk.
template <typename WT, int R>
__global__ __launch_bounds__(256) void bias_pack_kernel(const WT *W1, const int32_t *idx, int B, int V, uint4 *ep) {
    constexpr int C = 2 * PackedE<WT, R>::NF;  // chunks a row
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= B * C) return;
    const int b = t / C, c = t % C;
    const int row = min(max(idx[b], 0), V - 1);
    ep[size_t(b >> 5) * PackedE<WT, R>::BLOCK + PackedE<WT, R>::slot(b & 31, c)] =
        reinterpret_cast<const uint4 *>(W1 + size_t(row) * R)[c];
}


// bias_pair_lds with the A-fragment reads issued as inline asm, so that the
// compiler, which cannot tell one stage buffer's direct loads from another's,
// puts no wait for the stage loads in front of them; the caller has waited
// for the stage.  The reads run D K-steps ahead and each step waits for its
// own pair (LDS reads complete in order; any other lgkm operation in flight
// only lengthens the wait).  The wait is tied to the pair's registers, so the
// MFMAs that use them cannot move above it.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int R>
__device__ __forceinline__ void gemm_pair(const EFrags<uint16_t, R> &ef, const uint8_t *buf, int lane, f32x16_t &c0,
                                          f32x16_t &c1) {
    using L = TileLDS<uint16_t, R>;
    constexpr int S = EFrags<uint16_t, R>::S;
    constexpr int D = S < 3 ? S : 3;
    const int m = lane & 31, h = lane >> 5;
    const uint32_t row =
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t *)buf)) + m * L::RB;
    u32x4_t a0[D], a1[D];
    auto rd = [&](u32x4_t &x0, u32x4_t &x1, int s) __device__ {
        const uint32_t ad = row + L::chunk(m, 2 * s + h) * 16;
        asm volatile("ds_read_b128 %0, %1" : "=v"(x0) : "v"(ad));
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x1) : "v"(ad), "i"(L::BYTES));
    };
#pragma unroll
    for (int s = 0; s < D; ++s) rd(a0[s], a1[s], s);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        u32x4_t x0 = a0[s % D], x1 = a1[s % D];
        const int left = (S - s < D ? S - s : D) - 1;  // younger pairs in flight
        if (left == 2)
            asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(x0), "+v"(x1));
        else if (left == 1)
            asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(x0), "+v"(x1));
        else
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x0), "+v"(x1));
        if (s + D < S) rd(a0[s % D], a1[s % D], s + D);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x0),
                                                     __builtin_bit_cast(bf16x8_t, ef.e[s]), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x1),
                                                     __builtin_bit_cast(bf16x8_t, ef.e[s]), c1, 0, 0, 0);
    }
}
// f32 factors: the compiler-scheduled reads (it drains the stage loads first)
template <int R>
__device__ __forceinline__ void gemm_pair(const EFrags<float, R> &ef, const uint8_t *buf, int lane, f32x16_t &c0,
                                          f32x16_t &c1) {
    bias_pair_lds(ef, buf, lane, c0, c1);
}

// The draft step's tiling with its epilogue cut down to a running maximum: the
// same workgroups, two-tile W2 stages and MFMA chains, no U_k read and no
// sampling.  Without the U_k regions the LDS holds four stages, so three are
// in flight while one is consumed: each wave waits for its own direct loads
// of the stage (in-order vmcnt) and a bare barrier then covers every wave's,
// without the full drain that __syncthreads' release fence would force.
template <typename WT, int R>
__global__ __launch_bounds__(kStepThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bias_gemm_kernel(
    GemmParams p) {
    using L = TileLDS<WT, R>;
    using DMA = StageDMA<WT, R, kStepThreads>;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[2 * L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[2 * L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[2 * L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t lds3[2 * L::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = lg / p.nbg, bg = lg % p.nbg;
    const int bb = bg * (kStepThreads / 64) + wave;
    const bool wave_ok = bb < p.nbb;
    const int n = lane & 31, h = lane >> 5;
    const int b = bb * 32 + n;
    const bool row_ok = wave_ok && b < p.B;
    const WT *W2 = static_cast<const WT *>(p.W2);
    EFrags<WT, R> ef;
    if (wave_ok) ef.load_packed(p.ep + size_t(bb) * PackedE<WT, R>::BLOCK, lane);
    DMA dma;
    dma.init(tid);
    const int t_begin = chunk * p.tiles_per_chunk;
    const int t_end = min(p.ntiles, t_begin + p.tiles_per_chunk);
    const int nst = (t_end - t_begin + 1) >> 1;
    const bool tail = (t_begin + 2 * nst) * kTile > p.V;
    const int nfull = nst - (tail ? 1 : 0);
    float mx = kNegInf;
    auto stage = [&](const uint8_t *buf, int t0, bool masked) __device__ {
        f32x16_t c0 = {}, c1 = {};
        gemm_pair(ef, buf, lane, c0, c1);
        if (masked) {
            // value 4i+j of lane (n, h) is entry 8i + 4h + j of each tile
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (t0 * kTile + 8 * i + 4 * h + j >= p.V) c0[4 * i + j] = kNegInf;
                    if ((t0 + 1) * kTile + 8 * i + 4 * h + j >= p.V) c1[4 * i + j] = kNegInf;
                }
        }
        // the first level is an ordinary fmaxf, which the compiler orders
        // after the MFMAs that produce c0 and c1; max3f is inline asm and
        // must not read accumulators straight from the chain
        float d[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) d[e] = fmaxf(c0[e], c1[e]);
        float m0 = max3f(d[0], d[1], d[2]), m1 = max3f(d[3], d[4], d[5]);
#pragma unroll
        for (int e = 6; e < 14; e += 4) {
            m0 = max3f(m0, d[e], d[e + 1]);
            m1 = max3f(m1, d[e + 2], d[e + 3]);
        }
        mx = max3f(max3f(m0, d[14], d[15]), m1, mx);
    };
    auto v0_of = [&](int i) { return (t_begin + 2 * i) * kTile; };
    // stage i of the chunk: wait until its loads (and every older one) have
    // landed, join the workgroup, refill the buffer stage i - 1 used with
    // stage i + 3, consume stage i
    // (restrict: the compiler may then tell the refill's direct loads from the
    // buffer being read, and wait only for the older ones)
    auto step = [&](int i, const uint8_t *__restrict__ cur, uint8_t *__restrict__ refill) __device__ {
        const int after = min(2, nfull - 1 - i);  // younger stages in flight; uniform
        if (after == 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA::J));
        else if (after == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA::J));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        if (i + 3 < nfull) dma.template issue<false>(W2, v0_of(i + 3), p.V, refill, wave);
        if (wave_ok) stage(cur, t_begin + 2 * i, false);
    };
    if (nfull >= 3) {
        dma.template issue<false>(W2, v0_of(0), p.V, lds0, wave);
        dma.template issue<false>(W2, v0_of(1), p.V, lds1, wave);
        dma.template issue<false>(W2, v0_of(2), p.V, lds2, wave);
        // The loop's own loads write no registers and it reads the W1
        // fragments loaded before it, so the compiler would drain every load
        // at the loop entry, stages included.  Waiting for the fragments only
        // (they are older than the stages) and passing them through an empty
        // asm makes them plain register values to it.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * DMA::J));
        if (wave_ok) ef.pin();
        for (int i = 0; i < nfull; i += 4) {
            step(i, lds0, lds3);
            if (i + 1 >= nfull) break;
            step(i + 1, lds1, lds0);
            if (i + 2 >= nfull) break;
            step(i + 2, lds2, lds1);
            if (i + 3 >= nfull) break;
            step(i + 3, lds3, lds2);
        }
    } else {
        // one or two full stages: loaded together, then consumed
        if (nfull > 0) dma.template issue<false>(W2, v0_of(0), p.V, lds0, wave);
        if (nfull > 1) dma.template issue<false>(W2, v0_of(1), p.V, lds1, wave);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave_ok && nfull > 0) stage(lds0, t_begin, false);
        if (wave_ok && nfull > 1) stage(lds1, t_begin + 2, false);
    }
    if (tail) {
        __syncthreads();  // every wave is done with every buffer
        dma.template issue<true>(W2, v0_of(nfull), p.V, lds0, wave);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave_ok) stage(lds0, t_begin + 2 * nfull, true);
    }
    mx = fmaxf(mx, bfly<5>(mx));  // the two lane halves held different rows of the same tiles
    if (h == 0 && row_ok) p.pm[size_t(b) * p.nchunk + chunk] = mx;
}

// Row maxima from the per-chunk maxima: one wave per request.
__global__ __launch_bounds__(256) void bias_rowmax_kernel(const float *pm, int B, int nchunk, float *out) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= B) return;
    float m = kNegInf;
    for (int c = lane; c < nchunk; c += 64) m = fmaxf(m, pm[size_t(b) * nchunk + c]);
    bfly_steps<0, 6>([&](auto st) { m = fmaxf(m, bfly<decltype(st)::value>(m)); });
    if (lane == 0) out[b] = m;
}

template <typename WT, int R>
hipError_t launch_gemm_typed(const void *W1, const void *W2, const int32_t *idx, int B, int V, const DraftPlan &pl,
                             const DraftWork &w, float *rowmax, hipStream_t s) {
    // the rows packed first (the draft step's later positions get them from
    // the reduce), so that the product's time is the product alone
    constexpr int C = 2 * PackedE<WT, R>::NF;
    launch_kernel("bias_pack", (bias_pack_kernel<WT, R>), dim3((B * C + 255) / 256), dim3(256), s,
                  static_cast<const WT *>(W1), idx, B, V, w.ep);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmParams gp{w.ep, W2, B, V, pl.nbb, pl.nbg, pl.ntiles, pl.tiles_per_chunk, pl.nchunk, w.pm};
    launch_kernel("bias_gemm", (bias_gemm_kernel<WT, R>), dim3(pl.blocks), dim3(kStepThreads), s, gp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bias_rowmax_kernel, dim3((B + 3) / 4), dim3(256), 0, s, w.pm, B, pl.nchunk, rowmax);
    return hipGetLastError();
}

template <typename WT, int R>
hipError_t launch_typed(const DraftArgs &a, const DraftPlan &pl, const DraftWork &w, hipStream_t s) {
    const bool track2 = a.margin_out != nullptr;
    const bool vec = (reinterpret_cast<uintptr_t>(a.U) % 16 == 0) && (a.V % 4 == 0);
    const bool hvec = a.d % 4 == 0 && reinterpret_cast<uintptr_t>(a.hidden) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(a.conf_w) % 16 == 0;
    bool rnn = false;
    if constexpr (sizeof(WT) == 2) rnn = a.Wgco != nullptr;
    RnnProjPlan pp{};
    if (rnn) {
        // the h part of every position's gate product, before position 1
        pp = rnn_proj_plan(a.B, a.gamma, a.r, a.rnn_d);
        if (pp.S > 0 && w.rnn_yh) {
            const hipError_t e = launch_rnn_hproj(a.rnn_h, static_cast<const uint16_t *>(a.Wgco), w.rnn_yh, a.B,
                                                  a.gamma, a.r, a.rnn_d, pp, s);
            if (e != hipSuccess) return e;
        } else {
            pp.S = 0;
        }
    }
    for (int k = 1; k <= a.gamma; ++k) {
        const int32_t *xprev = (k == 1) ? a.anchor : a.x_out + (k - 2);
        const int xprev_stride = (k == 1) ? 1 : a.gamma;
        if (rnn) {
            // the RNN head's e_k replaces W1[x_{k-1}]: the step reads row
            // b * gamma + k - 1 of e_out as row rnn_idx[b] of e_out + (k - 1) r
            RnnGateArgs g{};
            g.s_in = (k == 1) ? nullptr : w.rnn_s[(k - 1) & 1];
            g.s_out = (k == a.gamma && a.state_out) ? a.state_out : w.rnn_s[k & 1];
            g.xprev = xprev;
            g.xprev_stride = xprev_stride;
            g.h = a.rnn_h + size_t(k - 1) * a.rnn_d;
            g.h_stride = size_t(a.gamma) * a.rnn_d;
            g.W1 = static_cast<const uint16_t *>(a.W1);
            g.Wgco = static_cast<const uint16_t *>(a.Wgco);
            g.e_out = a.e_out + size_t(k - 1) * a.r;
            g.e_stride = size_t(a.gamma) * a.r;
            g.idx_out = (k == 1) ? w.rnn_idx : nullptr;
            g.gamma = a.gamma;
            g.B = a.B;
            g.V = a.V;
            g.r = a.r;
            g.d = a.rnn_d;
            if (pp.S > 0) {
                g.yh = w.rnn_yh;
                g.yh_split = size_t(a.B) * a.gamma * 3 * a.r;
                g.yS = pp.S;
                g.kpos = k - 1;
            }
            const hipError_t e = launch_rnn_gate(g, s);
            if (e != hipSuccess) return e;
        }
        StepParams sp{};
        sp.U = a.U + size_t(k - 1) * a.V;
        sp.u_stride = size_t(a.gamma) * a.V;
        sp.W1 = rnn ? static_cast<const void *>(a.e_out + size_t(k - 1) * a.r) : a.W1;
        sp.W2 = a.W2;
        sp.xprev = rnn ? w.rnn_idx : xprev;
        sp.xprev_stride = rnn ? 1 : xprev_stride;
        sp.erows = rnn ? a.B * a.gamma : a.V;
        sp.temperature = a.temperature;
        sp.B = a.B;
        sp.V = a.V;
        sp.k = k;
        sp.key0 = a.key0;
        sp.key1 = a.key1;
        sp.round32 = a.round32;
        sp.nbb = pl.nbb;
        sp.nw = pl.nw;
        sp.nbg = pl.nbg;
        sp.ntiles = pl.ntiles;
        sp.tiles_per_chunk = pl.tiles_per_chunk;
        sp.nchunk = pl.nchunk;
        sp.vec = vec;
        sp.pm = w.pm;
        sp.ps = w.ps;
        sp.pb = w.pb;
        sp.p2 = w.p2;
        sp.pi = w.pi;
        // the Markov head's later positions take the rows the previous reduce packed
        const bool packed = !rnn && k > 1;
        sp.ep = w.ep;
        const dim3 grid(pl.blocks), block(kStepThreads);
        auto step = [&](auto t2, auto vc, auto pk) {
            launch_kernel("draft_step",
                          (draft_step_kernel<WT, R, decltype(t2)::value, decltype(vc)::value, decltype(pk)::value>),
                          grid, block, s, sp);
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        if (track2) {
            if (vec)
                packed ? step(T_{}, T_{}, T_{}) : step(T_{}, T_{}, F_{});
            else
                packed ? step(T_{}, F_{}, T_{}) : step(T_{}, F_{}, F_{});
        } else {
            if (vec)
                packed ? step(F_{}, T_{}, T_{}) : step(F_{}, T_{}, F_{});
            else
                packed ? step(F_{}, F_{}, T_{}) : step(F_{}, F_{}, F_{});
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;

        ReduceParams rp{};
        rp.U = sp.U;
        rp.u_stride = sp.u_stride;
        rp.W1 = sp.W1;
        rp.W2 = a.W2;
        rp.xprev = sp.xprev;
        rp.xprev_stride = sp.xprev_stride;
        rp.erows = sp.erows;
        rp.temperature = a.temperature;
        rp.B = a.B;
        rp.V = a.V;
        rp.k = k;
        rp.gamma = a.gamma;
        rp.nchunk = pl.nchunk;
        rp.ntiles = pl.ntiles;
        rp.key0 = a.key0;
        rp.key1 = a.key1;
        rp.round32 = a.round32;
        rp.pm = w.pm;
        rp.ps = w.ps;
        rp.pb = w.pb;
        rp.p2 = w.p2;
        rp.pi = w.pi;
        rp.x_out = a.x_out;
        rp.lse_out = a.lse_out;
        rp.qx_out = a.qx_out;
        rp.margin_out = a.margin_out;
        rp.ep_out = (!rnn && k < a.gamma) ? w.ep : nullptr;
        if (a.conf_out) {
            rp.hidden = a.hidden + size_t(k - 1) * a.d;
            rp.h_stride = size_t(a.gamma) * a.d;
            rp.conf_w = a.conf_w;
            rp.d = a.d;
            rp.hvec = hvec;
            rp.conf_tau = a.conf_tau;
            rp.conf_out = a.conf_out;
            rp.surv_out = a.surv_out;
            launch_kernel("draft_reduce", (draft_reduce_kernel<WT, R, true>), dim3((a.B + kReduceWaves - 1) / kReduceWaves),
                          dim3(64 * kReduceWaves), s, rp);
        } else {
            launch_kernel("draft_reduce", (draft_reduce_kernel<WT, R, false>), dim3((a.B + kReduceWaves - 1) / kReduceWaves),
                          dim3(64 * kReduceWaves), s, rp);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

DraftPlan tile_walk_plan(int B, int V, int nw_max, long long target_blocks, int align) {
    DraftPlan p{};
    p.nbb = (B + 31) / 32;
    p.nw = std::min(nw_max, p.nbb);
    p.nbg = (p.nbb + p.nw - 1) / p.nw;
    p.ntiles = (V + kTile - 1) / kTile;
    long long tpc = std::max<long long>(1, (1LL * p.ntiles * p.nbg + target_blocks - 1) / target_blocks);
    tpc = (tpc + align - 1) / align * align;
    p.tiles_per_chunk = int(std::min<long long>(tpc, (p.ntiles + align - 1) / align * align));
    p.nchunk = (p.ntiles + p.tiles_per_chunk - 1) / p.tiles_per_chunk;
    p.blocks = p.nchunk * p.nbg;
    return p;
}

DraftPlan draft_plan(int B, int V) {
    // 8-wave workgroups holding two 2-tile LDS stages (64 KB at bf16 rank 256)
    // and up to 256 registers a lane: one workgroup per CU, so about 256
    // workgroups; chunks are whole 2-tile stages
    return tile_walk_plan(B, V, kStepThreads / 64, 256, 2);
}

DraftWork draft_carve(void *ws, int B, const DraftPlan &p, size_t *bytes, int rnn_r, int rnn_gamma, int rnn_d) {
    Carve c(ws);
    const size_t n = size_t(B) * p.nchunk;
    DraftWork w{};
    w.pm = c.take<float>(n);
    w.ps = c.take<float>(n);
    w.pb = c.take<float>(n);
    w.p2 = c.take<float>(n);
    w.pi = c.take<int32_t>(n);
    // packed E rows of every request block, at the largest row size (512 bytes)
    w.ep = c.take<uint4>(size_t(p.nbb) * 32 * 32);
    if (rnn_r > 0) {
        w.rnn_s[0] = c.take<float>(size_t(B) * rnn_r);
        w.rnn_s[1] = c.take<float>(size_t(B) * rnn_r);
        w.rnn_idx = c.take<int32_t>(B);
        const RnnProjPlan pp = rnn_proj_plan(B, rnn_gamma, rnn_r, rnn_d);
        if (pp.S > 0) w.rnn_yh = c.take<float>(pp.floats);
    }
    if (bytes) *bytes = c.off + 256;
    return w;
}

hipError_t launch_bias_gemm(const void *W1, const void *W2, int wdtype, const int32_t *idx, int B, int V, int r,
                            const DraftPlan &p, const DraftWork &w, float *rowmax, hipStream_t s) {
    if (wdtype == 0) {
        switch (r) {
            case 16: return launch_gemm_typed<uint16_t, 16>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 32: return launch_gemm_typed<uint16_t, 32>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 64: return launch_gemm_typed<uint16_t, 64>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 128: return launch_gemm_typed<uint16_t, 128>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 256: return launch_gemm_typed<uint16_t, 256>(W1, W2, idx, B, V, p, w, rowmax, s);
        }
    } else {
        switch (r) {
            case 16: return launch_gemm_typed<float, 16>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 32: return launch_gemm_typed<float, 32>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 64: return launch_gemm_typed<float, 64>(W1, W2, idx, B, V, p, w, rowmax, s);
            case 128: return launch_gemm_typed<float, 128>(W1, W2, idx, B, V, p, w, rowmax, s);
        }
    }
    return hipErrorInvalidValue;
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
