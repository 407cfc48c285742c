// verify.hip -- the verify half of a DSpark round on gfx950: exact rejection
// sampling of the drafts against the target distributions, with ragged
// per-request verify lengths.
//
// Method ("DeepSeek DSpark explained" (share.concentrate1.com), section 05:
// accept x with probability min(1, p(x)/q(x)); on rejection draw from
// r(v) = max(p - q, 0) / sum max(p - q, 0); section 02: the first rejection
// discards the rest of the block, a bonus token follows when every draft
// passes, every request moves forward by at least one token; page
// "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io), sections 1 and 4.1
// for the same rule).  The draw from r (and from p for the bonus token) is a
// two-level Gumbel-max: a race over 32-entry vocabulary tiles by the log of
// their mass (Philox stream 4), then over the entries of the winning tile
// (stream 2).
//
// Kernels, in launch order:
//   verify_prep      1 workgroup, for batches above 512 requests (smaller
//                    ones have the walk or the first pass do it): packed row
//                    offsets (scan of 1 + ell, or the caller's, checked),
//                    output defaults, request state.
//   verify_walk      batches of 192 requests or more: one workgroup a
//                    request streams its rows in position order for
//                    logsumexp(t / T) in base 2 and the lowest-index argmax,
//                    decides each position right after its row (the accept
//                    test u*q < p, or a greedy request's bonus row) and stops
//                    at the first rejection, so no row past it is used.  A
//                    sampled request's bonus row is read by the draw only.
//   verify_tail      after the walk, for walked batches of at most 320
//                    requests and blocks of at least 4 drafts: the rows from
//                    the fourth on of the requests still accepting after row
//                    3, a workgroup a row, all at once; the last workgroup of
//                    a request to finish decides its positions in order.
//                    After the position passes instead of their last
//                    launches, when that saves launches and the rows it may
//                    read are few and cheap: it first decides the last pass's
//                    positions itself.
//   verify_pass      smaller batches, instead of the walk: one launch a
//                    position for the first few positions, one a pair of
//                    positions after them (from the first one on for a
//                    small batch), and a last one that only decides.  Each
//                    runs over the requests still testing: one wave per
//                    (request, row, vocabulary segment) first decides the
//                    positions the previous launch reduced, from the
//                    segment statistics it left (the accept test u*q < p,
//                    or the bonus row), then, if the request goes on,
//                    streams its segment of the row for logsumexp(t / T) in
//                    base 2 and the lowest-index argmax.  A request stops at
//                    its first rejection, so no row past it is read, except
//                    the second row of a pair.
//   verify_draw      level 1: every workgroup lists the drawing requests
//                    (residual draws first, bonus draws last, in request
//                    order); waves of 32 listed requests walk vocabulary
//                    chunks; residual rows recompute q_j with the draft's
//                    LDS-staged MFMA bias tile and sum max(p_j - q_j, 0) per
//                    tile, bonus rows take tile logsumexps of p; the tiles
//                    race with their noise.
//   verify_finish    level 2: one wave per drawing request merges the chunk
//                    partials, recomputes the winning tile's 32 entries and
//                    races them; writes the emitted token and S.  One more
//                    workgroup scans the emitted counts into out_offsets.
#include "device_common.hpp"
#include "dspark.h"
#include "internal.hpp"
#include "stage.hpp"

#include <algorithm>
#include <type_traits>

namespace dspark {

namespace {

constexpr int kStatusBadEll = 1;
constexpr int kStatusBadOffsets = 2;
constexpr int kStatusRowsOutOfRange = 4;

constexpr int kModeDone = 0;
constexpr int kModeResidual = 1;
constexpr int kModeBonus = 2;
constexpr int kPrepInKernelMaxBatch = 512;
constexpr int kPassRows = 2;  // row slots a position pass can hold

// v of the first active lane, as a scalar
__device__ __forceinline__ float uniform_f(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ float wave_sum(float v) {
    bfly_steps<0, 6>([&](auto st) { v += bfly<decltype(st)::value>(v); });
    return v;
}

__device__ __forceinline__ int wave_isum(int v) {
    bfly_steps<0, 6>([&](auto st) { v += bfly<decltype(st)::value>(v); });
    return v;
}

__device__ __forceinline__ void argmax_merge(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// value/index argmax across the wave: larger value, lower index on ties
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
    bfly_steps<0, 6>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float v2 = bfly<S>(v);
        const int i2 = bfly<S>(i);
        argmax_merge(v, i, v2, i2);
    });
}

// Exclusive scan over a workgroup of NT threads of one int per thread.
template <int NT>
__device__ int block_exclusive_scan(int v, int *lds, int *total) {
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

struct PrepParams {
    const int32_t *ell, *row_offsets;
    int B, gamma, n_target_rows;
    int32_t *off, *mode, *req_flags;
    int32_t *n_accept_out, *tokens_out;
    float *diag_out, *resid_out;
};

// Checks one request's ell and row offset (o: the computed offset, replaced by
// the caller's when given) and returns its input flags; *off_out gets the
// offset to use (0 for a request that fails).
__device__ __forceinline__ int check_request(const int32_t *ell, const int32_t *row_offsets, int b, int gamma,
                                             int n_target_rows, int o, int *off_out) {
    const int e_raw = ell[b];
    const int e = min(max(e_raw, 0), gamma);
    int f = (e_raw == e) ? 0 : kStatusBadEll;
    if (row_offsets) {
        o = row_offsets[b];
        const int o1 = row_offsets[b + 1];
        if (o < 0 || o1 - o != 1 + e_raw) f |= kStatusBadOffsets;
    }
    if (f == 0 && o + e + 1 > n_target_rows) f |= kStatusRowsOutOfRange;
    *off_out = f == 0 ? o : 0;
    return f;
}

// The output defaults of request b, shared by `stride` threads of which this
// is number `lane`.
__device__ __forceinline__ void output_defaults(int b, int gamma, int lane, int stride, int32_t *n_accept_out,
                                                int32_t *tokens_out, float *diag_out, float *resid_out) {
    int32_t *tok = tokens_out + size_t(b) * (gamma + 1);
    for (int i = lane; i <= gamma; i += stride) tok[i] = -1;
    if (diag_out)
        for (int i = lane; i < 2 * (gamma + 1); i += stride)
            diag_out[size_t(b) * 2 * (gamma + 1) + i] = __builtin_nanf("");
    if (lane == 0) {
        n_accept_out[b] = -1;  // set by the pass that ends the request
        if (resid_out) resid_out[b] = -1.f;
    }
}

// Input checks, row offsets and output defaults of a large batch, by one
// workgroup (a small batch has them done by its first position pass).
__global__ __launch_bounds__(1024) void verify_prep_kernel(PrepParams p) {
    __shared__ int lds[1024];
    const int t = threadIdx.x;
    const int seg = (p.B + 1023) / 1024;
    const int b0 = min(p.B, t * seg), b1 = min(p.B, b0 + seg);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += 1 + min(max(p.ell[b], 0), p.gamma);
    int total = 0;
    int base = block_exclusive_scan<1024>(local, lds, &total);
    // offsets: computed, or the caller's after a consistency check
    for (int b = b0; b < b1; ++b) {
        int o = 0;
        const int f = check_request(p.ell, p.row_offsets, b, p.gamma, p.n_target_rows, base, &o);
        p.off[b] = o;
        p.mode[b] = f == 0 ? kModeDone : -1;
        p.req_flags[b] = f;
        output_defaults(b, p.gamma, 0, 1, p.n_accept_out, p.tokens_out, p.diag_out, p.resid_out);
        base += 1 + min(max(p.ell[b], 0), p.gamma);
    }
    if (t == 1023) p.off[p.B] = p.row_offsets ? p.row_offsets[p.B] : total;
    // the status word is the OR of the requests' flags, formed by the finish
}

// Position k = j - 1 of request b, from its merged row statistics: the accept
// test (k <= ell) or the bonus row (k = ell + 1, greedy only).  A sampled
// request that accepts x_ell has its bonus outcome written at once.  Every
// workgroup of the request takes the same decision; only `writer` stores it.
// Returns whether the request goes on to position j.
// xk, qk: x_k and q_k(x_k) (any value when k > ell).  P: the position passes'
// or the walk's parameters (the same output fields).
template <class P>
__device__ bool pass_decide(const P &p, int b, int L, int k, bool sampled, float lse2, int amax, float tx2,
                            int xk, float qk, bool writer) {
    int32_t *tok = p.tokens_out + size_t(b) * (p.gamma + 1);
    bool bonus = false;
    if (k <= L) {
        bool acc;
        float pk, ratio;
        if (sampled) {
            pk = fast_exp2(tx2 - lse2);
            const float u = uniform01(scalar_word(kStreamAccept, k, uint32_t(b), p.round32, p.key0, p.key1));
            acc = u * qk < pk;
            ratio = qk > 0.f ? fminf(1.f, pk / qk) : 1.f;
        } else {
            acc = (xk == amax);
            pk = acc ? 1.f : 0.f;
            ratio = pk;
        }
        if (writer && p.diag_out) {
            p.diag_out[(size_t(b) * (p.gamma + 1) + (k - 1)) * 2 + 0] = pk;
            p.diag_out[(size_t(b) * (p.gamma + 1) + (k - 1)) * 2 + 1] = ratio;
        }
        if (acc) {
            if (writer) tok[k - 1] = xk;
            // a sampled request goes on only while a draft is left to test:
            // the draw takes its bonus token from row ell + 1 itself, and
            // that row's statistics are never used
            if (!sampled || k < L) return true;
            bonus = true;
            k = L + 1;
            lse2 = 0.f;
        }
        if (writer) p.n_accept_out[b] = bonus ? L : k - 1;
    } else {
        if (writer) p.n_accept_out[b] = L;
        bonus = true;
    }
    if (!writer) return false;
    p.jpos[b] = k;
    if (!sampled) {
        tok[k - 1] = amax;
        p.mode[b] = kModeDone;
        return false;
    }
    p.fin_lse2[b] = lse2;
    if (bonus) {
        p.mode[b] = kModeBonus;
    } else {
        p.mode[b] = kModeResidual;
        // what the residual draw needs to rebuild q_k
        p.prev[b] = p.erow_mode ? b * p.gamma + k - 1
                                : min(max(k == 1 ? p.anchor[b] : p.x[size_t(b) * p.gamma + k - 2], 0), p.V - 1);
        p.lse2q[b] = p.lse_q[size_t(b) * p.gamma + k - 1] * kLog2e;
    }
    return false;
}

// ------------------------------------------------------------------ position walk

// One workgroup walks one request's target rows in position order: it streams
// row j for the base-2 logsumexp of t / T (and the lowest-index argmax of a
// greedy row), decides position j from it (the accept test for j <= ell, the
// bonus row for j = ell + 1, which only a greedy request reads: a sampled
// one ends at x_ell, its bonus token drawn from the row by the draw) and goes
// on to row j + 1 only after an accepted draft, so no row past the first
// rejection is read.  The decision needs the
// whole row, and the whole row is this workgroup's: its waves meet once a row
// in LDS, and every wave merges the same statistics and takes the same
// decision, so no other workgroup and no fence is involved.  A batch fills
// the chip with one row a CU at first; the few requests still testing late in
// the block each stream a row at a CU's own load and exp2 rate.
// One wave a SIMD: with two a SIMD the arbiter favours the older wave, and
// a row's merge waited for the last wave (measured 2.4-3.3 us a row late in
// the block, 6 us on the first row).  Each lane keeps two batches of 16 float4
// groups.
constexpr int kWalkThreads = 256;
// batches from this size on are walked a workgroup a request (at 256 the walk
// and the position passes took the same time; at 64 and 32 requests, which
// leave most CUs idle, the passes were 1.7 and 2.3 times faster)
constexpr int kWalkMinBatch = 192;
constexpr int kWalkGroups = 16;
// third word of a raw buffer descriptor (dword data, no swizzle) on gfx9-family chips
constexpr int kBufferWord3 = 0x00020000;
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const float kconst_float;  // scalar-loadable (read-only) float
constexpr int kWalkWaves = kWalkThreads / 64;
static_assert(kWalkWaves <= 16, "the per-row merge runs over 16 lanes");

struct WalkParams {
    const float *target;
    const int32_t *x, *ell;
    const float *qx, *temperature;
    int B, gamma, V, vec;
    uint32_t key0, key1, round32;
    int32_t *off;
    // prep != 0: the walk also checks each request's inputs, forms its row
    // offset (a sum over ell) and writes the output defaults
    int prep, n_target_rows;
    const int32_t *row_offsets;
    int32_t *req_flags;
    float *resid_out;
    int32_t *mode, *jpos, *prev;
    float *fin_lse2, *lse2q;
    int erow_mode;  // 1: the residual's head row is row b * gamma + k - 1 of W1 (the head's rows)
    const int32_t *anchor;
    const float *lse_q;
    int32_t *n_accept_out, *tokens_out;
    float *diag_out;
    // tail_from > 0: a request still accepting when row tail_from is next
    // stops there (mode kModeTail, tail_flag 1) and the tail kernel reads
    // rows tail_from .. ell + 1; tail_* hold [B, gamma + 2 - tail_from] row
    // statistics and [B] counts of those rows reduced
    int tail_from;
    int32_t *tail_flag, *tail_cnt, *tail_amax;
    float *tail_lse2, *tail_tx;
    // tail_din > 0: the tail kernel follows the position passes instead of
    // the walk; the last pass reduced rows tail_from - tail_din ..
    // tail_from - 1 of the requests with act_in set and left their segment
    // statistics (as a pass's *_in buffers), which the tail kernel decides
    // first
    int tail_din, nseg_in, seg_stride;
    size_t row_stride;
    const int32_t *act_in, *pi_in;
    const float *pm_in, *ps_in, *pv_in, *tx_in;
};

// The walk leaves a request to the tail kernel (an intermediate mode, never
// seen by the draw)
constexpr int kModeTail = 3;
// rows from this one on are read by the tail kernel, for batches of at most
// kTailMaxBatch requests (more leave few CUs idle late in the block) and
// blocks of at least kTailMinGamma drafts
constexpr int kTailFrom = 4;
constexpr int kTailMaxBatch = 320;
constexpr int kTailMinGamma = 4;

// One batch of U float4 groups of a row into a thread's running base-2
// logsumexp (m, s) of x * sc; group u holds entries v0 + STRIDE u .. + 3 and
// counts only if valid(u).  The scale is positive, so the maximum is taken
// on the raw values and the scale folds into one fma per entry.  ARGMAX
// (greedy rows, sc = 1) also keeps the lowest-index maximum (av, ai).
template <bool ARGMAX, int U, int STRIDE, class Valid>
__device__ __forceinline__ void row_batch(float4 (&xs)[U], int v0, Valid valid, float sc, float &m, float &s, float &av,
                                          int &ai) {
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!valid(u)) xs[u] = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
        bm = fmaxf(fmaxf(bm, fmaxf(xs[u].x, xs[u].y)), fmaxf(xs[u].z, xs[u].w));
    }
    const float mn = fmaxf(m, bm * sc);
    if (mn != kNegInf) {
        const float nm = -mn;
        float add = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            add += fast_exp2(__builtin_fmaf(xs[u].x, sc, nm)) + fast_exp2(__builtin_fmaf(xs[u].y, sc, nm)) +
                   fast_exp2(__builtin_fmaf(xs[u].z, sc, nm)) + fast_exp2(__builtin_fmaf(xs[u].w, sc, nm));
        s = s * fast_exp2(m - mn) + add;
        m = mn;
    }
    if constexpr (ARGMAX) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float xv = f4get(xs[u], jj);
                if (xv > av) {
                    av = xv;
                    ai = v0 + STRIDE * u + jj;
                }
            }
    }
}

// One batch of U float4 groups into a thread's running base-2 logsumexp
// (m, s) of x * sc, the walk's form of row_batch: FULL batches lie inside the
// row (no masking); the maximum is taken with v_max3 on the raw values (the
// scale is positive), two entries an instruction.  ARGMAX (greedy rows,
// sc = 1) also keeps the lowest-index maximum; group u holds entries
// v0 + STRIDE u .. + 3.
template <bool ARGMAX, bool FULL, int U, int STRIDE>
__device__ __forceinline__ void walk_batch(float4 (&xs)[U], int v0, int nvalid_groups, float sc, float &m, float &s,
                                           float &av, int &ai) {
    static_assert(U % 2 == 0, "groups in pairs");
    if constexpr (!FULL) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u >= nvalid_groups) xs[u] = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
    }
    if constexpr (ARGMAX) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float xv = f4get(xs[u], jj);
                if (xv > av) {
                    av = xv;
                    ai = v0 + STRIDE * u + jj;
                }
            }
    }
    float b0 = max3f(xs[0].x, xs[0].y, xs[0].z), b1 = max3f(xs[0].w, xs[1].x, xs[1].y);
#pragma unroll
    for (int u = 1; u < U; u += 2) {
        b0 = max3f(b0, xs[u].z, xs[u].w);
        if (u + 1 < U) {
            b1 = max3f(b1, xs[u + 1].x, xs[u + 1].y);
            b0 = max3f(b0, xs[u + 1].z, xs[u + 1].w);
        }
    }
    const float mn = fmaxf(m, fmaxf(b0, b1) * sc);
    const float mg = (mn == kNegInf) ? 0.f : mn;  // an all -inf batch adds 2^-inf = 0
    const float nm = -mg;
    // every exponential first (independent), then a balanced sum
#pragma unroll
    for (int u = 0; u < U; ++u) {
        xs[u].x = fast_exp2(__builtin_fmaf(xs[u].x, sc, nm));
        xs[u].y = fast_exp2(__builtin_fmaf(xs[u].y, sc, nm));
        xs[u].z = fast_exp2(__builtin_fmaf(xs[u].z, sc, nm));
        xs[u].w = fast_exp2(__builtin_fmaf(xs[u].w, sc, nm));
    }
    float t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = (xs[u].x + xs[u].y) + (xs[u].z + xs[u].w);
#pragma unroll
    for (int w = 1; w < U; w *= 2)
#pragma unroll
        for (int u = 0; u + w < U; u += 2 * w) t[u] += t[u + w];
    s = __builtin_fmaf(s, fast_exp2(m - mg), t[0]);
    m = mn;
}

// The statistics of one row of V entries at trow (any alignment), reduced over
// the thread's share: entries t, t + NT, ...
template <bool ARGMAX>
__device__ __forceinline__ void walk_row_scalar(const float *trow, int V, float sc, float &m, float &s, float &av,
                                                int &ai) {
    for (int v = threadIdx.x; v < V; v += kWalkThreads) {
        const float xv = trow[v] * sc;
        const float mn = fmaxf(m, xv);
        if (mn != kNegInf) {
            s = s * fast_exp2(m - mn) + fast_exp2(xv - mn);
            m = mn;
        }
        if (ARGMAX && xv > av) {
            av = xv;
            ai = v;
        }
    }
}

// The workgroup's LDS for merging a row's statistics: a slot a wave, in two
// sets that alternate by row parity (the next row's writes never meet this
// row's reads).
struct WalkMergeLds {
    float m[2][kWalkWaves], s[2][kWalkWaves], v[2][kWalkWaves];
    int i[2][kWalkWaves];
};

// Row `par`'s statistics, complete in the threads' running states (m, s, av,
// ai), merged over the workgroup; the states are reset for the next row.
// Every wave merges the same statistics in the same order, and the results,
// the row's base-2 logsumexp lse2 and its lowest-index argmax amax, come out
// as scalars: the decision that follows is uniform to the compiler as well
// (scalar branches, exact load counts across the walk's loop).
__device__ __forceinline__ void walk_merge_row(WalkMergeLds &l, int par, int V, float &m, float &s, float &av,
                                               int &ai, float &lse2, int &amax) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bfly_steps<0, 6>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float m_o = bfly<S>(m), s_o = bfly<S>(s), v_o = bfly<S>(av);
        const int i_o = bfly<S>(ai);
        lse_merge(m, s, m_o, s_o);
        argmax_merge(av, ai, v_o, i_o);
    });
    if (lane == 0) {
        l.m[par][wave] = m;
        l.s[par][wave] = s;
        l.v[par][wave] = av;
        l.i[par][wave] = ai;
    }
    __syncthreads();
    float mm = kNegInf, ss = 0.f, vv = kNegInf;
    int ii = 0x7fffffff;
    if (lane < kWalkWaves) {
        mm = l.m[par][lane];
        ss = l.s[par][lane];
        vv = l.v[par][lane];
        ii = l.i[par][lane];
    }
    bfly_steps<0, 4>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float m_o = bfly<S>(mm), s_o = bfly<S>(ss), v_o = bfly<S>(vv);
        const int i_o = bfly<S>(ii);
        lse_merge(mm, ss, m_o, s_o);
        argmax_merge(vv, ii, v_o, i_o);
    });
    mm = uniform_f(mm);
    ss = uniform_f(ss);
    ii = __builtin_amdgcn_readfirstlane(ii);
    m = kNegInf;
    s = 0.f;
    av = kNegInf;
    ai = 0x7fffffff;
    lse2 = (mm == kNegInf) ? kNegInf : mm + fast_log2(ss);
    amax = min(max(ii, 0), V - 1);
}

// The test of draft position j from its target row's statistics (the accept
// rule of "DeepSeek DSpark explained", section 05): a sampled row accepts x_j when u q(x_j) < p(x_j), with
// p(x_j) = 2^(txs - lse2) (txs = t(x_j) log2(e) / T) and thr = u q(x_j); a
// greedy row accepts when x_j is the row's argmax.  pk and ratio get the
// position's diagnostics p(x_j) and min(1, p / q).
__device__ __forceinline__ bool position_test(bool sampled, float txs, float lse2, int amax, int xj, float qk,
                                              float thr, float &pk, float &ratio) {
    if (sampled) {
        pk = fast_exp2(txs - lse2);
        ratio = qk > 0.f ? fminf(1.f, pk / qk) : 1.f;
        return thr < pk;
    }
    const bool acc = xj == amax;
    pk = acc ? 1.f : 0.f;
    ratio = pk;
    return acc;
}

// Streams a request's rows j_first, j_first + 1, ... (row j at
// target + (offb + j - 1) V, V a multiple of 4, rows 16-byte aligned) into
// the threads' running statistics and calls finish(j) once row j is complete
// in them; the stream goes on to row j + 1 while finish returns true, and
// finish must return false at j_last.
//
// One pipeline over the batches of consecutive rows: thread t takes float4
// groups t, t + NT, ... of each batch of NT U groups (a fixed share, so the
// sums are formed in the same order on every run).  Two batches are in
// flight, so the first batch of row j + 1 goes out before position j is
// decided (and is dropped when the stream stops there): the loads do not
// drain at a row boundary.  A batch past j_last gets an empty buffer
// descriptor: it is issued like the others (the counts of loads in flight are
// the same on every path) but touches no memory.  The row and batch of each
// buffer are tracked as scalar counters.
template <class Finish>
__device__ __forceinline__ void walk_stream_rows(const float *target, int offb, int V, int j_first, int j_last,
                                                 bool sampled, float sc, float &m, float &s, float &av, int &ai,
                                                 Finish &&finish) {
    constexpr int U = kWalkGroups, NB = kWalkThreads * U;
    const int tid = threadIdx.x;
    const int n4 = V >> 2;
    const int nbr = (n4 + NB - 1) / NB;  // batches a row
    const int last_qb = (nbr - 1) * NB;  // first group of a row's last batch
    // Buffer loads: the row is a scalar descriptor whose range check returns
    // 0 past its end (masked when reduced), and a group's offset is the
    // thread's fixed part plus a scalar one, so a batch needs no address
    // registers of its own.
    const int voff = tid * 16;
    auto load = [&](float4(&xs)[U], int j, int qb) __device__ {
        const bool any = j <= j_last;  // uniform
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(target + size_t(offb + (any ? j : j_first) - 1) * V), 0, any ? n4 * 16 : 0,
            kBufferWord3);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const v4f_t x =
                __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (qb + kWalkThreads * u) * 16, kStreamPolicy);
            xs[u] = make_float4(x[0], x[1], x[2], x[3]);
        }
    };
    auto consume = [&](float4(&xs)[U], int qb) __device__ {
        if (qb + NB <= n4) {  // uniform: a full batch
            if (sampled)
                walk_batch<false, true, U, 4 * kWalkThreads>(xs, 4 * (qb + tid), U, sc, m, s, av, ai);
            else
                walk_batch<true, true, U, 4 * kWalkThreads>(xs, 4 * (qb + tid), U, sc, m, s, av, ai);
        } else {
            const int nv = (n4 - qb - tid + kWalkThreads - 1) / kWalkThreads;  // this thread's groups in the row
            if (sampled)
                walk_batch<false, false, U, 4 * kWalkThreads>(xs, 4 * (qb + tid), nv, sc, m, s, av, ai);
            else
                walk_batch<true, false, U, 4 * kWalkThreads>(xs, 4 * (qb + tid), nv, sc, m, s, av, ai);
        }
    };
    // (row, first group) of the batch in each buffer
    int ja = j_first, qa = 0, jb, qb;
    auto advance = [&](int j, int q, int &jn, int &qn) {
        if (q == last_qb) {
            jn = j + 1;
            qn = 0;
        } else {
            jn = j;
            qn = q + NB;
        }
    };
    float4 xa[U], xb[U];
    load(xa, ja, qa);
    for (;;) {
        advance(ja, qa, jb, qb);
        load(xb, jb, qb);
        consume(xa, qa);
        if (qa == last_qb && !finish(ja)) break;
        advance(jb, qb, ja, qa);
        load(xa, ja, qa);
        consume(xb, qb);
        if (qb == last_qb && !finish(jb)) break;
    }
}

__global__ __launch_bounds__(kWalkThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void verify_walk_kernel(
    WalkParams p) {
    __shared__ WalkMergeLds s_mg;
    __shared__ int s_x[DSPARK_MAX_GAMMA];
    __shared__ float s_q[DSPARK_MAX_GAMMA], s_thr[DSPARK_MAX_GAMMA];
    __shared__ float s_dp[DSPARK_MAX_GAMMA], s_dr[DSPARK_MAX_GAMMA];  // p_k(x_k), min(1, p/q) of tested positions
    __shared__ int s_off, s_mode;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float T = p.temperature[b];
    const int L_raw = p.ell[b];
    const bool sampled = T > 0.f;
    if (wave == 0) {
        // the request's state: its row offset and input checks (in the walk
        // for a small batch), its drafts, q(x) and accept thresholds u q
        int offb, md;
        if (p.prep) {
            int rows_before = 0;
            if (!p.row_offsets)
                for (int i = lane; i < b; i += 64) rows_before += 1 + min(max(p.ell[i], 0), p.gamma);
            const int o_cmp = wave_isum(rows_before);
            const int f = check_request(p.ell, p.row_offsets, b, p.gamma, p.n_target_rows, o_cmp, &offb);
            md = f == 0 ? kModeDone : -1;
            if (lane == 0) {
                p.off[b] = offb;
                p.req_flags[b] = f;
                if (b == p.B - 1)
                    p.off[p.B] = p.row_offsets ? p.row_offsets[p.B] : o_cmp + 1 + min(max(L_raw, 0), p.gamma);
            }
            output_defaults(b, p.gamma, lane, 64, p.n_accept_out, p.tokens_out, p.diag_out, p.resid_out);
        } else {
            offb = p.off[b];
            md = p.mode[b];
        }
        if (lane < p.gamma) {
            const size_t o = size_t(b) * p.gamma + lane;
            const float q = p.qx[o];
            s_x[lane] = p.x[o];
            s_q[lane] = q;
            // u q < p is the accept test; u q is formed here once
            s_thr[lane] = sampled ? uniform01(scalar_word(kStreamAccept, lane + 1, uint32_t(b), p.round32, p.key0,
                                                          p.key1)) * q
                                  : 0.f;
        }
        if (lane == 0) {
            s_off = offb;
            s_mode = md;
        }
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_mode) < 0) {  // failed its input checks: outputs keep their defaults
        if (tid == 0) {
            p.mode[b] = -1;
            if (p.tail_from) p.tail_flag[b] = 0;
        }
        return;
    }
    const int offb = __builtin_amdgcn_readfirstlane(s_off);
    const int L = L_raw;  // in [0, gamma] once the checks passed
    // the last row the request may need: a sampled request's bonus token is
    // drawn from row ell + 1 by the draw, which uses none of its statistics
    const int jl = sampled ? L : L + 1;
    const float sc = sampled ? kLog2e / T : 1.0f;
    auto row_of = [&](int j) { return p.target + size_t(offb + j - 1) * p.V; };
    // the thread's state for the current row: running base-2 logsumexp and
    // argmax (greedy)
    float m = kNegInf, s = 0.f, av = kNegInf;
    int ai = 0x7fffffff;
    // t(x_j) / T of the row being read, for its accept test: a scalar load
    // (through the constant address space; the rows are read-only here),
    // issued when the row starts and counted apart from the row's vector loads
    float txs = kNegInf;
    auto locate_x = [&](int j) {
        if (sampled && j <= L) {
            const int q = min(max(__builtin_amdgcn_readfirstlane(s_x[j - 1]), 0), p.V - 1);
            txs = reinterpret_cast<const kconst_float *>(reinterpret_cast<uintptr_t>(row_of(j)))[q] * sc;
        }
    };
    // the walk's outcome, the same in every thread; no global store is made
    // before the walk ends (the outputs go out after it); a sampled request
    // with no draft to test is a bonus draw without a row read
    int r_n = 0, r_j = 1, r_mode = jl == 0 ? kModeBonus : kModeDone, r_tok = -1;
    float r_lse2 = 0.f;
    // Row j is complete in the threads' states: merge it over the workgroup
    // and decide position j.  Returns whether the walk goes on to row j + 1
    // (with its t(x_j) load issued).
    auto finish_row = [&](int j) -> bool {
        float lse2;
        int amax;
        walk_merge_row(s_mg, j & 1, p.V, m, s, av, ai, lse2, amax);
        if (j <= L) {
            float pk, ratio;
            const bool acc =
                position_test(sampled, txs, lse2, amax, __builtin_amdgcn_readfirstlane(s_x[j - 1]),
                              uniform_f(s_q[j - 1]), uniform_f(s_thr[j - 1]), pk, ratio);
            if (tid == 0) {
                s_dp[j - 1] = pk;
                s_dr[j - 1] = ratio;
            }
            if (acc) {
                if (j == jl) {  // sampled, every draft accepted: the bonus draw
                    r_n = L;
                    r_j = L + 1;
                    r_mode = kModeBonus;
                    return false;
                }
                if (j + 1 != p.tail_from) {
                    locate_x(j + 1);
                    return true;
                }
                r_n = j;  // the later rows go to the tail kernel
                r_j = j + 1;
                r_mode = kModeTail;
                return false;
            }
            r_n = j - 1;  // first rejection at j: the residual draw (sampled) or the target's argmax (greedy)
            r_mode = sampled ? kModeResidual : kModeDone;
        } else {
            r_n = L;  // greedy, every draft accepted: the bonus token is row ell + 1's argmax
            r_mode = kModeDone;
        }
        r_j = j;
        r_lse2 = lse2;
        r_tok = amax;
        return false;
    };
    locate_x(1);
    if (!p.vec) {
        for (int j = 1; j <= jl; ++j) {
            if (sampled)
                walk_row_scalar<false>(row_of(j), p.V, sc, m, s, av, ai);
            else
                walk_row_scalar<true>(row_of(j), p.V, sc, m, s, av, ai);
            if (!finish_row(j)) break;
        }
    } else if (jl > 0) {
        walk_stream_rows(p.target, offb, p.V, 1, jl, sampled, sc, m, s, av, ai, finish_row);
    }
    if (tid == 0) {
        // the outcome: accepted drafts, the first rejection's or the bonus
        // row's data for the draw, diagnostics of every tested position (a
        // request left to the tail kernel: its accepted drafts and their
        // diagnostics so far)
        const bool tail = r_mode == kModeTail;
        int32_t *tok = p.tokens_out + size_t(b) * (p.gamma + 1);
        for (int k = 1; k <= r_n; ++k) tok[k - 1] = s_x[k - 1];
        if (!sampled && !tail) tok[r_j - 1] = r_tok;
        if (p.diag_out)
            for (int k = 1; k <= (tail ? r_n : min(r_j, L)); ++k) {
                p.diag_out[(size_t(b) * (p.gamma + 1) + (k - 1)) * 2 + 0] = s_dp[k - 1];
                p.diag_out[(size_t(b) * (p.gamma + 1) + (k - 1)) * 2 + 1] = s_dr[k - 1];
            }
        p.n_accept_out[b] = r_n;
        p.jpos[b] = r_j;
        p.mode[b] = r_mode;
        if (p.tail_from) {
            p.tail_flag[b] = tail ? 1 : 0;
            if (tail) p.tail_cnt[b] = 0;
        }
        if (sampled && !tail) p.fin_lse2[b] = r_lse2;
        if (r_mode == kModeResidual) {
            p.prev[b] = p.erow_mode ? b * p.gamma + r_j - 1
                                    : min(max(r_j == 1 ? p.anchor[b] : s_x[r_j - 2], 0), p.V - 1);
            p.lse2q[b] = p.lse_q[size_t(b) * p.gamma + r_j - 1] * kLog2e;
        }
    }
}

// ------------------------------------------------------------------ a block's last rows (after the walk or the passes)

// Rows tail_from .. ell + 1 (.. ell for a sampled request, whose bonus row
// only the draw reads) of the requests the walk left at row tail_from, a
// workgroup a row, all at once: a request's later rows are read whether or
// not an earlier one rejects (the rows past its first rejection are reduced
// and left unused), so the block's last rows take about one row's time
// instead of one each, on CUs the walk has left idle.  A row is streamed and
// merged by the walk's own code, so its statistics have the walk's bits.
// Each workgroup stores its row's statistics and counts itself in with one
// device-scope atomic (release); the one that counts its request's last row
// in (acquire) decides the request's positions in order, as the walk would,
// and writes its outcome.  No workgroup waits for another.  Workgroup
// s nt + t takes row tail_from + t of the s-th request of the batch with
// tail_flag set (nt = gamma + 2 - tail_from).
// After the position passes (tail_din > 0) the requests are those the last
// pass reduced rows for, and each workgroup first decides that pass's
// positions from its segment statistics, as the next pass would (workgroup
// t = 0 writes the outcome); a request that stops there reads no more rows.
__global__ __launch_bounds__(kWalkThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void verify_tail_kernel(
    WalkParams p) {
    static_assert(kTailFrom >= 2, "the walk decides row 1");
    __shared__ WalkMergeLds s_mg;
    __shared__ int s_go;
    __shared__ uint64_t s_ball[(kTailMaxBatch + 63) / 64];
    // every request's length, row offset, temperature and draft at this
    // workgroup's position, loaded with the flags (one round trip)
    __shared__ int s_rq_ell[kTailMaxBatch], s_rq_off[kTailMaxBatch], s_rq_x[kTailMaxBatch];
    __shared__ float s_rq_T[kTailMaxBatch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nt = p.gamma + 2 - p.tail_from;
    const int slot = blockIdx.x / nt, t = blockIdx.x - slot * nt;
    const int j = p.tail_from + t;
    const int nch = (p.B + 63) / 64;
    for (int c = wave; c < nch; c += kWalkWaves) {
        const int bq = c * 64 + lane;
        int fl = 0;
        if (bq < p.B) {
            fl = p.tail_din ? p.act_in[bq] : p.tail_flag[bq];
            s_rq_ell[bq] = p.ell[bq];
            s_rq_off[bq] = p.off[bq];
            s_rq_T[bq] = p.temperature[bq];
            s_rq_x[bq] = j <= p.gamma ? p.x[size_t(bq) * p.gamma + j - 1] : 0;
        }
        const uint64_t bal = __ballot(fl != 0);
        if (lane == 0) s_ball[c] = bal;
    }
    __syncthreads();
    int b = -1;
    {
        int rem = slot;
        for (int c = 0; c < nch; ++c) {
            uint64_t bal = s_ball[c];
            const int pc = __popcll(bal);
            if (rem < pc) {
                for (int i = 0; i < rem; ++i) bal &= bal - 1;
                b = c * 64 + __builtin_ctzll(bal);
                break;
            }
            rem -= pc;
        }
    }
    b = __builtin_amdgcn_readfirstlane(b);
    if (b < 0) return;
    const int L = __builtin_amdgcn_readfirstlane(s_rq_ell[b]);  // checked by the walk or the first pass
    const float T = uniform_f(s_rq_T[b]);
    const bool sampled = T > 0.f;
    const float sc = sampled ? kLog2e / T : 1.0f;
    const int jl = sampled ? L : L + 1;  // the request's last row (as in the walk)
    if (p.tail_din) {  // uniform
        if (j > jl && t > 0) return;
        if (wave == 0) {
            // the last pass's segment statistics, 64 / din lanes a row slot
            // (neutral where a lane holds none), merged within each group
            const int din = p.tail_din, lps = 64 / din;
            const int hq = min(lane / lps, din - 1), c = min(lane % lps, p.nseg_in - 1);
            const size_t o_in = hq * p.row_stride + size_t(b) * p.seg_stride + c;
            float mm = p.pm_in[o_in], s2 = p.ps_in[o_in], v2 = p.pv_in[o_in];
            int i2 = p.pi_in[o_in];
            float tx2[kPassRows], qk[kPassRows];
            int xk[kPassRows];
#pragma unroll
            for (int u = 0; u < kPassRows; ++u) {
                const int k = min(max(p.tail_from - din + u, 1), p.gamma);  // position decided from slot u (clamped)
                tx2[u] = p.tx_in[size_t(min(u, din - 1)) * p.B + b];
                xk[u] = p.x[size_t(b) * p.gamma + k - 1];
                qk[u] = p.qx[size_t(b) * p.gamma + k - 1];
            }
            if (!((lane / lps) < din && (lane % lps) < p.nseg_in)) {
                mm = kNegInf;
                s2 = 0.f;
                v2 = kNegInf;
                i2 = 0x7fffffff;
            }
            auto step = [&](auto st) {
                constexpr int S = decltype(st)::value;
                const float m_o = bfly<S>(mm), s_o = bfly<S>(s2), v_o = bfly<S>(v2);
                const int i_o = bfly<S>(i2);
                lse_merge(mm, s2, m_o, s_o);
                argmax_merge(v2, i2, v_o, i_o);
            };
            bfly_steps<0, 5>(step);
            if (din == 1) step(std::integral_constant<int, 5>{});
            float lse2[kPassRows];
            int amax[kPassRows];
#pragma unroll
            for (int u = 0; u < kPassRows; ++u) {
                const float mu = __shfl(mm, lps * min(u, din - 1)), su = __shfl(s2, lps * min(u, din - 1));
                lse2[u] = (mu == kNegInf) ? kNegInf : mu + fast_log2(su);
                amax[u] = min(max(__shfl(i2, lps * min(u, din - 1)), 0), p.V - 1);
            }
            int go_on = 0;
            if (lane == 0) {
                go_on = 1;
                for (int u = 0; u < din; ++u) {
                    const int k = p.tail_from - din + u;
                    if (!go_on || k > L + 1) break;
                    go_on = pass_decide(p, b, L, k, sampled, lse2[u], amax[u], tx2[u], xk[u], qk[u], t == 0);
                }
                s_go = go_on;
            }
        }
        __syncthreads();
        if (!__builtin_amdgcn_readfirstlane(s_go)) return;
    }
    if (j > jl) return;
    const int offb = __builtin_amdgcn_readfirstlane(s_rq_off[b]);
    float txs = kNegInf;
    if (sampled && j <= L) {
        const int q = min(max(__builtin_amdgcn_readfirstlane(s_rq_x[b]), 0), p.V - 1);
        txs = reinterpret_cast<const kconst_float *>(
                  reinterpret_cast<uintptr_t>(p.target + size_t(offb + j - 1) * p.V))[q] *
              sc;
    }
    // The decision's inputs, loaded while the row streams: in wave 0, lane i
    // takes the request's row tail_from + i (its draft, q(x), log-normaliser
    // of q, and the draft before it)
    const int jj = p.tail_from + lane;
    const bool row = wave == 0 && jj <= L + 1;
    int xj = -1, xprev = 0;
    float qk = 0.f, lq = 0.f;
    if (row) {
        const size_t ox = size_t(b) * p.gamma + jj - 1;
        xprev = p.x[ox - 1];
        if (jj <= L) {
            xj = p.x[ox];
            qk = p.qx[ox];
            lq = p.lse_q[ox];
        }
    }
    float m = kNegInf, s = 0.f, av = kNegInf;
    int ai = 0x7fffffff;
    float lse2 = 0.f;
    int amax = 0;
    walk_stream_rows(p.target, offb, p.V, j, j, sampled, sc, m, s, av, ai, [&](int jr) -> bool {
        walk_merge_row(s_mg, jr & 1, p.V, m, s, av, ai, lse2, amax);
        return false;
    });
    if (wave != 0) return;
    int last = 0;
    if (lane == 0) {
        const size_t o = size_t(b) * nt + t;
        p.tail_lse2[o] = lse2;
        p.tail_amax[o] = amax;
        p.tail_tx[o] = txs;
        last = __hip_atomic_fetch_add(p.tail_cnt + b, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
               jl - p.tail_from;  // the request's other rows (jl + 1 - tail_from in all) are in
    }
    if (!__builtin_amdgcn_readfirstlane(last)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // every position's test at once, then the first that stops (a
    // rejection, else the bonus row ell + 1, read for a greedy request only)
    float l2 = 0.f, pk = 0.f, ratio = 0.f;
    int am = 0;
    bool acc = false;
    if (row && jj <= jl) {
        const size_t o = size_t(b) * nt + lane;
        l2 = __hip_atomic_load(p.tail_lse2 + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        am = __hip_atomic_load(p.tail_amax + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float tx = __hip_atomic_load(p.tail_tx + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (jj <= L) {
            const float thr =
                sampled ? uniform01(scalar_word(kStreamAccept, jj, uint32_t(b), p.round32, p.key0, p.key1)) * qk
                        : 0.f;
            acc = position_test(sampled, tx, l2, am, xj, qk, thr, pk, ratio);
        }
    }
    const uint64_t stop = __ballot(row && (jj > L || !acc));  // lane ell + 1 - tail_from is set
    const int jf = p.tail_from + __builtin_ctzll(stop);
    int32_t *tok = p.tokens_out + size_t(b) * (p.gamma + 1);
    if (row && jj < jf) tok[jj - 1] = xj;
    if (p.diag_out && row && jj <= min(jf, L)) {
        p.diag_out[(size_t(b) * (p.gamma + 1) + (jj - 1)) * 2 + 0] = pk;
        p.diag_out[(size_t(b) * (p.gamma + 1) + (jj - 1)) * 2 + 1] = ratio;
    }
    if (jj == jf) {
        const bool rej = jf <= L;
        const int r_mode = !sampled ? kModeDone : (rej ? kModeResidual : kModeBonus);
        if (!sampled) tok[jf - 1] = am;
        p.n_accept_out[b] = rej ? jf - 1 : L;
        p.jpos[b] = jf;
        p.mode[b] = r_mode;
        if (sampled) p.fin_lse2[b] = l2;
        if (r_mode == kModeResidual) {
            p.prev[b] = p.erow_mode ? b * p.gamma + jf - 1 : min(max(xprev, 0), p.V - 1);
            p.lse2q[b] = lq * kLog2e;
        }
    }
}

// ------------------------------------------------------------------ position passes (small batches)

// Rows a position pass reduces: one or two consecutive positions of the
// requests still testing; the pass first decides the positions the previous
// pass reduced.  A request that rejects at the first of a pair has the second
// row read for nothing, against one launch less.  Few requests are still
// testing late in the block, so there the launch costs more than the row:
// the first kSinglePasses positions get a pass each, the rest go in pairs
// (an odd one left first on its own), then one pass decides the last rows.
// A batch whose rows at one position take at most kPairAllBytes pairs from
// the first position on: a launch costs about 7 us, about 45 MB of reads,
// against at most B V 4 bytes read for nothing a pair.
constexpr int kSinglePasses = 3;
// The position passes hand a block's last rows, at most kPassTailRows of
// them, to the tail kernel when that saves at least kPassTailLaunches
// launches (the last, decide-only pass included) and the rows it may read
// are few (at most kPassTailReads, about one a CU) and cheap: small rows
// (at most kPassTailSmallV entries), or rows late in the block, after at
// least kPassTailAfter passes, where few requests are still testing.  A
// launch costs about 4-5 us even with nothing to read; the tail kernel about
// 7 us, plus one row's time at a CU's read rate for the requests it reads.
constexpr int kPassTailRows = 4;
constexpr int kPassTailLaunches = 3;
constexpr int kPassTailReads = 256;
constexpr int kPassTailSmallV = 65536;
constexpr int kPassTailAfter = 3;
constexpr size_t kPairAllBytes = size_t(64) << 20;
// segments of a row in the first position pass and in the later ones
// (measured at the headline size: 8 first-pass segments take 1 us less than
// 4; 16 or 64 later segments take 1-2 us a pass more than 32)
constexpr int kSegFirst = 8, kSegLater = 32;
static_assert(kSegFirst <= 64 / kPassRows && kSegLater <= 64 / kPassRows,
              "the next pass merges a row's segment statistics in 64 / kPassRows lanes");

struct PassParams {
    const float *target;
    const int32_t *x, *ell;
    const float *qx, *temperature;
    int B, gamma, V, j0, vec;  // j0: first position this pass reduces
    int nseg, seg_len;  // this pass's segments of a row
    int nseg_in;        // the previous pass's
    int seg_stride;     // partials per request in the buffers
    size_t row_stride;  // partials per row slot of a pass (B * seg_stride)
    uint32_t key0, key1, round32;
    int32_t *off;
    // prep != 0 (first pass of a small batch): the pass also checks each
    // request's inputs, computes its row offset and writes the output defaults
    int prep, n_target_rows;
    const int32_t *row_offsets;
    int32_t *req_flags;
    float *resid_out;
    // pass p reads what pass p - 1 left and writes into the other half of
    // each double buffer; slot q holds the pass's q-th row
    const int32_t *act_in;  // [B] 1: the request's rows of the previous pass were reduced
    const float *pm_in, *ps_in, *pv_in, *tx_in;
    const int32_t *pi_in;
    int32_t *act_out;
    float *pm_out, *ps_out, *pv_out, *tx_out;
    int32_t *pi_out;
    int32_t *mode, *jpos, *prev;
    float *fin_lse2, *lse2q;
    int erow_mode;  // 1: the residual's head row is row b * gamma + k - 1 of W1 (the head's rows)
    const int32_t *anchor;
    const float *lse_q;
    int32_t *n_accept_out, *tokens_out;
    float *diag_out;
    int32_t *tail_cnt;  // non-null: the first pass zeroes each request's count for the tail kernel
};

// Pass p, one wave per (request, row slot q < DOUT, vocabulary segment),
// four requests to a workgroup.  First the request's DIN previous positions are
// decided, in order, from the segment statistics pass p - 1 wrote; a request
// that goes on streams segment sg of its row j0 + q: every lane keeps its own
// running max / sum of exp2 and argmax over batches of eight float4 loads,
// two batches in flight (one is reduced while the next lands), and the wave
// merges them.  The waves never wait for one another.  FIRST: the first pass,
// which decides nothing.
template <bool FIRST, int DIN, int DOUT>
__global__ __launch_bounds__(256) void verify_pass_kernel(PassParams p) {
    static_assert(DIN >= 1 && DIN <= kPassRows && DOUT >= 1 && DOUT <= kPassRows,
                  "row slots: the previous pass's (DIN) and this pass's (DOUT)");
    constexpr int LPS = 64 / DIN;  // lanes holding one previous row slot's segment statistics
    constexpr int LOG_LPS = DIN == 1 ? 6 : 5;
    const int sg = blockIdx.x % p.nseg;
    const int q = (blockIdx.x / p.nseg) % DOUT;
    const int b = (blockIdx.x / (p.nseg * DOUT)) * 4 + (threadIdx.x >> 6);
    const int j0 = p.j0, j = j0 + q;
    const int lane = threadIdx.x & 63;
    if (b >= p.B) return;
    const bool writer = sg == 0 && q == 0;
    int mode, offb, act, L;
    float T;
    float mm = kNegInf, s2 = 0.f, v2 = kNegInf;
    int i2 = 0x7fffffff;
    float tx2[DIN], qk[DIN];
    int xk[DIN];
    if constexpr (FIRST) {
        // the first pass decides nothing: it needs the request's temperature
        // and length and, for a small batch, does its input checks (the row
        // offset is a wave sum over ell, read in the same round)
        T = p.temperature[b];
        L = p.ell[b];
        act = 1;
        if (p.prep) {  // uniform
            int rows_before = 0;
            if (!p.row_offsets)
                for (int i = lane; i < b; i += 64) rows_before += 1 + min(max(p.ell[i], 0), p.gamma);
            const int o_cmp = wave_isum(rows_before);
            const int f = check_request(p.ell, p.row_offsets, b, p.gamma, p.n_target_rows, o_cmp, &offb);
            mode = f == 0 ? kModeDone : -1;
            if (writer) {
                if (lane == 0) {
                    p.off[b] = offb;
                    p.mode[b] = mode;
                    p.req_flags[b] = f;
                    if (p.tail_cnt) p.tail_cnt[b] = 0;
                    if (b == p.B - 1)
                        p.off[p.B] = p.row_offsets ? p.row_offsets[p.B] : o_cmp + 1 + min(max(L, 0), p.gamma);
                }
                output_defaults(b, p.gamma, lane, 64, p.n_accept_out, p.tokens_out, p.diag_out, p.resid_out);
            }
        } else {
            mode = p.mode[b];
            offb = p.off[b];
        }
    } else {
        // every load the decisions need, issued together and unconditionally
        // (clamped indices; what a case does not use is masked after): lane
        // group h (of LPS lanes) holds the segment statistics of the previous
        // pass's row slot h, read whatever the request's state
        const int hq = min(lane / LPS, DIN - 1), c = min(lane % LPS, p.nseg_in - 1);
        const size_t o_in = hq * p.row_stride + size_t(b) * p.seg_stride + c;
        mode = p.mode[b];
        offb = p.off[b];
        act = p.act_in[b];
        T = p.temperature[b];
        L = p.ell[b];
        mm = p.pm_in[o_in];
        s2 = p.ps_in[o_in];
        v2 = p.pv_in[o_in];
        i2 = p.pi_in[o_in];
#pragma unroll
        for (int u = 0; u < DIN; ++u) {
            const int k = min(max(j0 - DIN + u, 1), p.gamma);  // position decided from slot u (clamped)
            tx2[u] = p.tx_in[size_t(u) * p.B + b];
            xk[u] = p.x[size_t(b) * p.gamma + k - 1];
            qk[u] = p.qx[size_t(b) * p.gamma + k - 1];
        }
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::"v"(mode), "v"(offb), "v"(act), "v"(T), "v"(L), "v"(mm), "v"(s2), "v"(v2), "v"(i2));
        if (!((lane / LPS) < DIN && (lane % LPS) < p.nseg_in)) {
            mm = kNegInf;
            s2 = 0.f;
            v2 = kNegInf;
            i2 = 0x7fffffff;
        }
    }
    if (mode < 0 || act == 0) {
        if (writer && lane == 0) p.act_out[b] = 0;
        return;
    }
    const bool sampled = T > 0.f;
    const float sc = sampled ? kLog2e / T : 1.0f;
    if (!FIRST && j0 > 1) {
        bfly_steps<0, LOG_LPS>([&](auto st) {  // within each lane group
            constexpr int S = decltype(st)::value;
            const float m_o = bfly<S>(mm), s_o = bfly<S>(s2), v_o = bfly<S>(v2);
            const int i_o = bfly<S>(i2);
            lse_merge(mm, s2, m_o, s_o);
            argmax_merge(v2, i2, v_o, i_o);
        });
        float lse2[DIN];
        int amax[DIN];
#pragma unroll
        for (int u = 0; u < DIN; ++u) {
            const float mu = __shfl(mm, LPS * u), su = __shfl(s2, LPS * u);
            lse2[u] = (mu == kNegInf) ? kNegInf : mu + fast_log2(su);
            amax[u] = min(max(__shfl(i2, LPS * u), 0), p.V - 1);
        }
        int go_on = 0;
        if (lane == 0) {
            go_on = 1;
#pragma unroll
            for (int u = 0; u < DIN; ++u) {
                const int k = j0 - DIN + u;
                if (!go_on || k > L + 1) break;
                go_on = pass_decide(p, b, L, k, sampled, lse2[u], amax[u], tx2[u], xk[u], qk[u], writer);
            }
        }
        if (!__shfl(go_on, 0)) {
            if (writer && lane == 0) p.act_out[b] = 0;
            return;
        }
    }
    // the last row the request may need: a sampled request's bonus token is
    // drawn from row ell + 1 by the draw, which uses none of its statistics
    const int jl = sampled ? L : L + 1;
    if (j > jl) {  // no row at this slot (slot 0 has one once the request goes on, but in the first pass)
        if (writer && lane == 0) {
            p.act_out[b] = 0;
            if (FIRST) {  // sampled with no draft to test: the bonus draw, no row read
                p.n_accept_out[b] = 0;
                p.jpos[b] = 1;
                p.mode[b] = kModeBonus;
                p.fin_lse2[b] = 0.f;
            }
        }
        return;
    }
    const float *trow = p.target + size_t(offb + j - 1) * p.V;
    const int v_lo = sg * p.seg_len, v_hi = min(p.V, v_lo + p.seg_len);
    float m = kNegInf, s = 0.f, av = kNegInf;
    int ai = 0x7fffffff;
    if (p.vec) {
        // two batches of U float4 a lane, one in flight while the other is
        // reduced
        const float4 *r4 = reinterpret_cast<const float4 *>(trow);
        const int q_hi = v_hi >> 2;
        constexpr int U = 8;
        // loads past the segment re-read its last group and are masked when used
        auto load = [&](float4(&xs)[U], int qb) __device__ {
#pragma unroll
            for (int u = 0; u < U; ++u) xs[u] = load_stream(r4 + min(qb + lane + 64 * u, q_hi - 1));
        };
        // sampled rows keep no argmax (only greedy decisions use it); the
        // request, and so the branch, is uniform across the wave
        auto consume = [&](float4(&xs)[U], int qb) __device__ {
            auto valid = [&](int u) { return qb + lane + 64 * u < q_hi; };
            if (sampled)
                row_batch<false, U, 256>(xs, 4 * (qb + lane), valid, sc, m, s, av, ai);
            else
                row_batch<true, U, 256>(xs, 4 * (qb + lane), valid, sc, m, s, av, ai);
        };
        // The loop body is straight-line, so that every consume sees the
        // same loads in flight on every path into it; it runs while the
        // batch after the pair exists, and the last one or two batches
        // follow it.  The batch bounds are uniform across the wave.
        constexpr int NB = 64 * U;  // float4 groups a batch
        const int qs = v_lo >> 2;
        float4 xa[U], xb[U];
        load(xa, qs);
        int qb = qs;
        for (; qb + 2 * NB < q_hi; qb += 2 * NB) {
            load(xb, qb + NB);
            consume(xa, qb);
            load(xa, qb + 2 * NB);
            consume(xb, qb + NB);
        }
        if (qb + NB < q_hi) {
            load(xb, qb + NB);
            consume(xa, qb);
            consume(xb, qb + NB);
        } else {
            consume(xa, qb);
        }
    } else {
        for (int v = v_lo + lane; v < v_hi; v += 64) {
            const float xv = trow[v] * sc;
            const float mn = fmaxf(m, xv);
            if (mn != kNegInf) {
                s = s * fast_exp2(m - mn) + fast_exp2(xv - mn);
                m = mn;
            }
            if (xv > av) {
                av = xv;
                ai = v;
            }
        }
    }
    bfly_steps<0, 6>([&](auto st) {
        constexpr int S = decltype(st)::value;
        const float m_o = bfly<S>(m), s_o = bfly<S>(s), v_o = bfly<S>(av);
        const int i_o = bfly<S>(ai);
        lse_merge(m, s, m_o, s_o);
        argmax_merge(av, ai, v_o, i_o);
    });
    if (lane == 0) {
        const size_t o = q * p.row_stride + size_t(b) * p.seg_stride + sg;
        p.pm_out[o] = m;
        p.ps_out[o] = s;
        p.pv_out[o] = av;
        p.pi_out[o] = ai;
        if (writer) p.act_out[b] = 1;
        // t(x_j) for the accept test at j, from the segment that holds x_j
        if (sampled && j <= L) {
            const int xj = min(max(p.x[size_t(b) * p.gamma + j - 1], 0), p.V - 1);
            if (xj >= v_lo && xj < v_hi) p.tx_out[size_t(q) * p.B + b] = trow[xj] * sc;
        }
    }
}

// ------------------------------------------------------------------ draw

struct DrawParams {
    const float *U, *target;
    const void *W1, *W2;
    const int32_t *anchor, *x;
    const float *lse_q, *temperature;
    int B, gamma, V;
    int nbg, ntiles, tiles_per_chunk, nchunk;
    uint32_t key0, key1, round32;
    const int32_t *mode, *jpos, *off, *prev;
    const float *fin_lse2, *lse2q;
    float *dw_sum, *dw_bl;
    int32_t *dw_bt;
};

// The draw list, in request order: residual draws at entries [0, nres), bonus
// draws at [B - nbon, B).  Every workgroup forms it from the requests' modes
// (wave ballots over blocks of 64 requests, block counts in LDS) and keeps the
// NE entries from e0 on in lreq (-1 for none); scratch holds 2 ceil(B / 64) +
// NE ints.  Ends with a workgroup barrier.
template <int NW>
__device__ void build_draw_list(const int32_t *mode, int B, int e0, int NE, int *scratch, int &nres, int &nbon,
                                int *&lreq) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = (B + 63) / 64;
    int *cr = scratch, *cb = scratch + nch;
    lreq = scratch + 2 * nch;
    for (int i = tid; i < NE; i += NW * 64) lreq[i] = -1;
    for (int c = wave; c < nch; c += NW) {
        const int bq = c * 64 + lane;
        const int md = bq < B ? mode[bq] : kModeDone;
        const uint64_t br = __ballot(md == kModeResidual), bb = __ballot(md == kModeBonus);
        if (lane == 0) {
            cr[c] = __popcll(br);
            cb[c] = __popcll(bb);
        }
    }
    __syncthreads();
    int tr = 0, tb = 0;
    for (int i = lane; i < nch; i += 64) {
        tr += cr[i];
        tb += cb[i];
    }
    nres = wave_isum(tr);
    nbon = wave_isum(tb);
    const uint64_t below = (uint64_t(1) << lane) - 1;
    for (int c = wave; c < nch; c += NW) {
        int pr = 0, pb = 0;  // draws of each kind in the blocks before block c
        for (int i = lane; i < c; i += 64) {
            pr += cr[i];
            pb += cb[i];
        }
        pr = wave_isum(pr);
        pb = wave_isum(pb);
        const int bq = c * 64 + lane;
        const int md = bq < B ? mode[bq] : kModeDone;
        const uint64_t br = __ballot(md == kModeResidual), bb = __ballot(md == kModeBonus);
        int e = -1;
        if (md == kModeResidual) e = pr + __popcll(br & below);
        if (md == kModeBonus) e = B - nbon + pb + __popcll(bb & below);
        if (e >= e0 && e < e0 + NE) lreq[e - e0] = bq;
    }
    __syncthreads();
}

constexpr int kDrawThreads = 512;  // 8 waves: one block of 32 listed requests each
// A batch of at most two 32-request blocks draws with 2-wave workgroups
// instead: their stages take 64 KB of LDS, so two workgroups share a CU and
// the walk spreads over about 512 of them, where an 8-wave workgroup would
// hold one busy wave and the LDS of seven idle ones.
constexpr int kDrawSmallWaves = 2;

// Level 1 of the resample / bonus draws.  A workgroup of 8 waves walks the
// tiles of one vocabulary chunk, one tile per stage, each wave holding 32
// listed requests.  Every stage is double buffered in LDS and loaded by
// direct loads one stage ahead: the tile's W2 rows (shared by the workgroup)
// and, in wave-private regions, the requests' target rows p_j and (residual
// waves) U_j rows.  Residual waves recompute the q_j logits U_j + B_j of the
// tile with the draft's MFMA tile and sum max(p_j - q_j, 0) over it; bonus
// waves take the tile logsumexp of p.  Either way the tile score takes its
// noise from stream 4.  The two halves of a wave hold the two halves of the
// tile and combine their sums with one lane-half exchange.
template <typename WT, int R, bool VEC, int NWV>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(NWV >= 4 ? 2 : 1, 2))) void verify_draw_kernel(
    DrawParams p) {
    using L = TileLDS<WT, R>;
    using TR = TileRows<VEC>;
    __shared__ __attribute__((aligned(16))) uint8_t ldsW0[L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsW1[L::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsU0[NWV * TR::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsU1[NWV * TR::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsT0[NWV * TR::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ldsT1[NWV * TR::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = lg / p.nbg, bg = lg % p.nbg;
    const int e0 = bg * NWV * 32;  // first list entry of the workgroup
    const int t_begin = chunk * p.tiles_per_chunk;
    const int t_end = min(p.ntiles, t_begin + p.tiles_per_chunk);
    const bool tail = t_end * kTile > p.V;  // the chunk's last tile runs past the vocabulary
    const int nfull = (t_end - t_begin) - (tail ? 1 : 0);
    const WT *W2 = static_cast<const WT *>(p.W2);
    TileDMA<WT, R, NWV * 64> dma;
    dma.init(tid);
    // the first W2 tile needs no list: it goes out first (and is only wasted
    // by a workgroup that holds no residual draw)
    if (nfull > 0) dma.template issue<false>(W2, t_begin * kTile, p.V, ldsW0, wave);
    // entries [0, nres) of the draw list are residual draws, [B - nbon, B)
    // bonus draws; the two never overlap, so at most one wave holds both kinds.
    // The list is built in the second target buffer, which the first stage
    // leaves free.
    int nres, nbon, *lreq;
    build_draw_list<NWV>(p.mode, p.B, e0, NWV * 32, reinterpret_cast<int *>(ldsT1), nres, nbon, lreq);
    const int bon0 = p.B - nbon;  // first bonus entry
    if (e0 >= nres && (nbon == 0 || e0 + NWV * 32 <= bon0 || e0 >= p.B)) {
        __builtin_amdgcn_s_waitcnt(0);  // the whole workgroup is idle: its direct loads land before it leaves
        return;
    }
    const bool need_w2 = e0 < nres;  // uniform across the workgroup
    const int w0 = e0 + wave * 32;   // first entry of the wave
    const bool wave_resid = w0 < nres;                          // uniform across the wave
    const bool wave_bonus = w0 < p.B && w0 + 32 > bon0 && nbon > 0;  // uniform across the wave
    const bool wave_ok = wave_resid || wave_bonus;
    const int n = lane & 31, h = lane >> 5;
    const int e = w0 + n;
    const bool resid = e < nres;
    const bool ok = resid || (e >= bon0 && e < p.B);
    const int req = ok ? max(lreq[wave * 32 + n], 0) : 0;
    const int j = wave_ok ? p.jpos[req] : 1;
    const float sc = wave_ok ? kLog2e / p.temperature[req] : 1.0f;
    const float lse2t = wave_ok ? p.fin_lse2[req] : 0.f;
    const int trow_i = ok ? p.off[req] + j - 1 : -1;  // packed target row

    EFrags<WT, R> ef;
    int urow_i = -1;  // row of U
    float lse2q = 0.f;
    if (wave_resid) {
        ef.load(static_cast<const WT *>(p.W1) + size_t(resid ? p.prev[req] : 0) * R, h);
        if (resid) {
            urow_i = req * p.gamma + j - 1;
            lse2q = p.lse2q[req];
        }
    }
    TR su, stg;
    if (wave_ok) stg.init(lane, p.target, size_t(p.V), [&](int r) { return __shfl(trow_i, r); });
    if (wave_resid) su.init(lane, p.U, size_t(p.V), [&](int r) { return __shfl(urow_i, r); });
    const int roff = wave * TR::BYTES;  // this wave's region in each region buffer

    float S = 0.f;  // residual mass (both halves hold the same sum)
    float best = kNegInf;
    int bt = t_begin;
    uint4 tw = make_uint4(0u, 0u, 0u, 0u);

    auto issue = [&](int t, uint8_t *w, uint8_t *ur, uint8_t *tr, auto clamp, bool with_w2 = true) __device__ {
        constexpr bool C = decltype(clamp)::value;
        if (need_w2 && with_w2) dma.template issue<C>(W2, t * kTile, p.V, w, wave);
        if (wave_ok) stg.template issue<C>(t * kTile, p.V, tr + roff, lane);
        if (wave_resid) su.template issue<C>(t * kTile, p.V, ur + roff, lane);
    };
    auto stage = [&](int t, const uint8_t *w, const uint8_t *ur, const uint8_t *tr, bool masked) __device__ {
        f32x16_t pv = stg.read(tr + roff, lane);
        f32x16_t c;
        if (wave_resid) c = bias_tile_lds(ef, w, lane, su.read(ur + roff, lane));
        if (masked) {
            // value 4i+jj of lane (n, h) is entry 8i + 4h + jj of the tile
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (t * kTile + 8 * i + 4 * h + jj >= p.V) pv[4 * i + jj] = c[4 * i + jj] = kNegInf;
        }
        if (t == t_begin || (t & 3) == 0)
            tw = noise_block(kStreamResampleTile, j, uint32_t(t) >> 2, uint32_t(req), p.round32, p.key0, p.key1);
        const float g = gumbel2(u4get(tw, t & 3));
        // a wave holding both kinds scores the tile both ways and each lane
        // keeps its own, so the lane-half exchanges never run divergent
        float Lt = kNegInf, rt = 0.f;
        if (wave_resid) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                r0 += fmaxf(fast_exp2(__builtin_fmaf(pv[e], sc, -lse2t)) - fast_exp2(__builtin_fmaf(c[e], sc, -lse2q)),
                            0.f);
                r1 += fmaxf(fast_exp2(__builtin_fmaf(pv[e + 1], sc, -lse2t)) -
                                fast_exp2(__builtin_fmaf(c[e + 1], sc, -lse2q)),
                            0.f);
            }
            rt = half_sum(r0 + r1);
            Lt = rt > 0.f ? fast_log2(rt) + g : kNegInf;
        }
        if (wave_bonus) {
            float mh = max3f(pv[0], pv[1], pv[2]);
#pragma unroll
            for (int e = 3; e < 15; e += 2) mh = max3f(mh, pv[e], pv[e + 1]);
            mh = max3f(mh, pv[15], pv[15]) * sc;
            const float mt = half_max(mh);
            const float mg = (mt == kNegInf) ? 0.f : mt;
            float sh = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) sh += fast_exp2(__builtin_fmaf(pv[e], sc, -mg));
            const float st = half_sum(sh);
            if (!resid) Lt = mg + fast_log2(st) + g;
        }
        if (resid) S += rt;
        if (Lt > best) {
            best = Lt;
            bt = t;
        }
    };

    using NoClamp = std::integral_constant<bool, false>;
    using Clamp = std::integral_constant<bool, true>;
    if (nfull > 0) issue(t_begin, ldsW0, ldsU0, ldsT0, NoClamp{}, false);  // its W2 tile is out already
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
    if (h == 0 && ok) {
        const size_t o = size_t(req) * p.nchunk + chunk;  // by request: the finish needs no list
        p.dw_sum[o] = S;
        p.dw_bl[o] = best;
        p.dw_bt[o] = bt;
    }
}

// ------------------------------------------------------------------ finish

struct FinishParams {
    const float *U, *target;
    const void *W1, *W2;
    const int32_t *anchor, *x;
    const float *lse_q, *temperature;
    int B, gamma, V, nchunk, ntiles;
    uint32_t key0, key1, round32;
    int32_t *status;
    const int32_t *mode, *n_accept, *off, *jpos, *prev, *req_flags;
    const float *fin_lse2, *lse2q;
    const float *dw_sum, *dw_bl;
    const int32_t *dw_bt;
    int32_t *tokens_out, *out_offsets;
    float *resid_out;
};

// Winner of an entry race held by the 32 lower lanes of the wave.
__device__ __forceinline__ int wave_race(float score, int v) {
    float s = (threadIdx.x & 32) ? kNegInf : score;
    int i = v;
    wave_argmax(s, i);
    return i;
}

// Level 2 of the draws, and the emitted token: one wave per drawing request.
// Exclusive scan of the emitted counts n_b + 1 (0 for a request that failed
// its check) into out_offsets, by one workgroup of 256 threads.
__device__ void scan_out_offsets(const FinishParams &p) {
    __shared__ int lds[256];
    const int t = threadIdx.x;
    const int seg = (p.B + 255) / 256;
    const int b0 = min(p.B, t * seg), b1 = min(p.B, b0 + seg);
    int local = 0;
    for (int b = b0; b < b1; ++b)
        if (p.mode[b] >= 0) local += p.n_accept[b] + 1;
    int total = 0;
    int e = block_exclusive_scan<256>(local, lds, &total);
    for (int b = b0; b < b1; ++b) {
        p.out_offsets[b] = e;
        if (p.mode[b] >= 0) e += p.n_accept[b] + 1;
    }
    if (t == 0) p.out_offsets[p.B] = total;
}

// The status word: the OR of every request's input flags, by one workgroup.
__device__ void status_word(const FinishParams &p) {
    __shared__ int flags;
    if (threadIdx.x == 0) flags = 0;
    __syncthreads();
    int local = 0;
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) local |= p.req_flags[b];
    if (local) atomicOr(&flags, local);
    __syncthreads();
    if (threadIdx.x == 0) p.status[0] = flags;
}

template <typename WT, int R>
__global__ __launch_bounds__(256) void verify_finish_kernel(FinishParams p) {
    if (blockIdx.x == gridDim.x - 1) {  // the extra workgroup
        status_word(p);
        if (p.out_offsets) scan_out_offsets(p);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= p.B) return;
    // the request's state and its first batch of chunk partials (kept by
    // request) in one round of loads, read whatever the mode (used only by
    // drawing requests); the W1 row and the winning tile's entries follow in
    // a second
    constexpr int PC = 4;
    float cs[PC], cb[PC];
    int ct[PC];
    auto load_batch = [&](int c0) __device__ {
#pragma unroll
        for (int u = 0; u < PC; ++u) {
            const int c = c0 + lane + 64 * u;  // past the chunks: re-reads chunk 0, masked below
            const size_t o = size_t(b) * p.nchunk + (c < p.nchunk ? c : 0);
            cs[u] = p.dw_sum[o];
            cb[u] = p.dw_bl[o];
            ct[u] = p.dw_bt[o];
        }
    };
    const int mode = p.mode[b];
    const int j = p.jpos[b], off = p.off[b], prev = p.prev[b];
    const float T = p.temperature[b], lse2t = p.fin_lse2[b], lse2q_in = p.lse2q[b];
    load_batch(0);
    // an empty use ahead of the branch keeps the compiler from sinking the
    // loads after it, which would put another round trip on the path
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"v"(j), "v"(off), "v"(prev), "v"(T), "v"(lse2t), "v"(lse2q_in));
    asm volatile("" ::"v"(cs[0]), "v"(cs[1]), "v"(cs[2]), "v"(cs[3]), "v"(cb[0]), "v"(cb[1]), "v"(cb[2]),
                 "v"(cb[3]), "v"(ct[0]), "v"(ct[1]), "v"(ct[2]), "v"(ct[3]));
    if (mode != kModeResidual && mode != kModeBonus) return;
    const float sc = kLog2e / T;
    const float *trow = p.target + size_t(off + j - 1) * p.V;
    RowHalf<WT, R> w1;
    float lse2q = 0.f;
    if (mode == kModeResidual) {
        w1.load(static_cast<const WT *>(p.W1) + size_t(prev) * R, lane >> 5);
        lse2q = lse2q_in;
    }
    float S = 0.f, bl = kNegInf;
    int tile = 0x7fffffff;
    for (int c0 = 0; c0 < p.nchunk; c0 += 64 * PC) {
        if (c0 > 0) load_batch(c0);
#pragma unroll
        for (int u = 0; u < PC; ++u) {
            if (c0 + lane + 64 * u < p.nchunk) {
                S += cs[u];
                argmax_merge(bl, tile, cb[u], ct[u]);
            }
        }
    }
    S = wave_sum(S);
    wave_argmax(bl, tile);

    const int i = lane & 31, h = lane >> 5;
    const bool use_res = mode == kModeResidual && S > 0.f && bl > kNegInf;
    if (mode == kModeResidual && !use_res) {
        // p and q agree to rounding: draw from p_j, level 1 over every tile here
        float b1 = kNegInf;
        int t1 = 0x7fffffff;
        for (int t = lane; t < p.ntiles; t += 64) {
            const int v0 = t * kTile, v1 = min(p.V, v0 + kTile);
            float mm = kNegInf;
            for (int v = v0; v < v1; ++v) mm = fmaxf(mm, trow[v] * sc);
            if (mm == kNegInf) continue;
            float ss = 0.f;
            for (int v = v0; v < v1; ++v) ss += fast_exp2(trow[v] * sc - mm);
            const float g =
                gumbel2(noise_word(kStreamResampleTile, j, uint32_t(t), uint32_t(b), p.round32, p.key0, p.key1));
            argmax_merge(b1, t1, mm + fast_log2(ss) + g, t);
        }
        wave_argmax(b1, t1);
        tile = t1;
    }
    tile = min(max(tile, 0), p.ntiles - 1);
    const int v = tile * kTile + i;
    const bool valid = v < p.V;
    const int vc = min(v, p.V - 1);
    const float g = gumbel2(noise_word(kStreamResample, j, uint32_t(vc), uint32_t(b), p.round32, p.key0, p.key1));
    const float tt = trow[vc] * sc;
    float score;
    if (use_res) {
        const float u_v = p.U[(size_t(b) * p.gamma + j - 1) * p.V + vc];
        const float d = w1.dot(static_cast<const WT *>(p.W2) + size_t(vc) * R, h);
        const float logit = u_v + d;
        const float q = fast_exp2(__builtin_fmaf(logit, sc, -lse2q));
        const float pv = fast_exp2(tt - lse2t);
        const float res = fmaxf(pv - q, 0.f);
        score = res > 0.f ? fast_log2(res) + g : kNegInf;
    } else {
        score = tt + g;
    }
    if (!valid) score = kNegInf;
    const int y = min(max(wave_race(score, v), 0), p.V - 1);
    if (lane == 0) {
        p.tokens_out[size_t(b) * (p.gamma + 1) + j - 1] = y;
        if (p.resid_out && mode == kModeResidual) p.resid_out[b] = S;
    }
}

// The position passes of a block of gamma: first row and row count of each
// (`single` single rows, then pairs, an odd row left over first), then
// the decide-only pass (rows 0 at j0 = gamma + 2).
struct PassRows {
    int j0, rows;
};
int pass_schedule(int gamma, int single, PassRows *out) {
    int n = 0, j = 1;
    const int last = gamma + 1;
    for (; j <= last && j <= single; ++j) out[n++] = {j, 1};
    if ((last - j + 1) % 2 == 1 && j <= last) out[n++] = {j++, 1};
    for (; j <= last; j += 2) out[n++] = {j, 2};
    out[n++] = {last + 1, 0};
    return n;
}

template <typename WT, int R>
hipError_t launch_typed(const VerifyArgs &a, const VerifyPlan &pl, const VerifyWork &w, hipStream_t s) {
    hipError_t e;
    // a small batch has its input checks and output defaults done by the
    // walk (each workgroup forms its request's row offset from ell, O(B)
    // reads); a large one by a workgroup of its own
    const bool prep_in_kernel = a.B <= kPrepInKernelMaxBatch;
    if (!prep_in_kernel) {
        PrepParams pp{a.ell, a.row_offsets, a.B, a.gamma, a.n_target_rows, w.off,
                      w.mode, w.req_flags, a.n_accept_out, a.tokens_out, a.diag_out, a.resid_out};
        launch_kernel("verify_prep", verify_prep_kernel, dim3(1), dim3(1024), s, pp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool vec_t = (reinterpret_cast<uintptr_t>(a.target) % 16 == 0) && (a.V % 4 == 0);
    const bool vec_u = (reinterpret_cast<uintptr_t>(a.U) % 16 == 0) && (a.V % 4 == 0);
    // the walk's parameters; the tail kernel takes them too
    auto walk_params = [&]() {
        WalkParams w_{};
        w_.target = a.target;
        w_.x = a.x;
        w_.ell = a.ell;
        w_.qx = a.qx;
        w_.temperature = a.temperature;
        w_.B = a.B;
        w_.gamma = a.gamma;
        w_.V = a.V;
        w_.vec = vec_t;
        w_.key0 = a.key0;
        w_.key1 = a.key1;
        w_.round32 = a.round32;
        w_.off = w.off;
        w_.prep = prep_in_kernel ? 1 : 0;
        w_.n_target_rows = a.n_target_rows;
        w_.row_offsets = a.row_offsets;
        w_.req_flags = w.req_flags;
        w_.resid_out = a.resid_out;
        w_.mode = w.mode;
        w_.jpos = w.jpos;
        w_.prev = w.prev;
        w_.fin_lse2 = w.fin_lse2;
        w_.lse2q = w.lse2q;
        w_.erow_mode = a.erow_mode;
        w_.anchor = a.anchor;
        w_.lse_q = a.lse_q;
        w_.n_accept_out = a.n_accept_out;
        w_.tokens_out = a.tokens_out;
        w_.diag_out = a.diag_out;
        w_.tail_flag = w.tail_flag;
        w_.tail_cnt = w.tail_cnt;
        w_.tail_amax = w.tail_amax;
        w_.tail_lse2 = w.tail_lse2;
        w_.tail_tx = w.tail_tx;
        return w_;
    };
    if (pl.walk) {
        WalkParams wp = walk_params();
        // the tail kernel streams rows the vector way only, and finds its
        // requests among at most kTailMaxBatch
        wp.tail_from = (vec_t && a.B <= kTailMaxBatch) ? pl.tail_from : 0;
        launch_kernel("verify_walk", verify_walk_kernel, dim3(a.B), dim3(kWalkThreads), s, wp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (wp.tail_from) {
            const int nt = a.gamma + 2 - wp.tail_from;
            launch_kernel("verify_tail", verify_tail_kernel, dim3(size_t(a.B) * nt), dim3(kWalkThreads), s, wp);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        PassRows sched[DSPARK_MAX_GAMMA + 2];  // gamma is checked at the boundary
        const int single = size_t(a.B) * a.V * sizeof(float) <= kPairAllBytes ? 0 : kSinglePasses;
        int npass = pass_schedule(a.gamma, single, sched);
        // the block's last rows, after the first pass that qualifies, go to
        // the tail kernel (rows streamed the vector way, requests found among
        // at most kTailMaxBatch, each request's tail count zeroed by the
        // first pass's input checks)
        int tail_from = 0, tail_din = 0;
        if (vec_t && prep_in_kernel && a.B <= kTailMaxBatch)
            for (int i = 0; i < npass && sched[i].rows > 0; ++i) {
                const int jn = sched[i].j0 + sched[i].rows, left = a.gamma + 2 - jn;
                if (left >= 1 && left <= kPassTailRows && npass - (i + 1) >= kPassTailLaunches &&
                    a.B * left <= kPassTailReads && (a.V <= kPassTailSmallV || i + 1 >= kPassTailAfter)) {
                    npass = i + 1;
                    tail_from = jn;
                    tail_din = sched[i].rows;
                    break;
                }
            }
        const size_t rs = size_t(a.B) * pl.nseg_max;  // one row slot
        const size_t half = rs * kPassRows;
        for (int pass = 1; pass <= npass; ++pass) {
            const int in = (pass - 1) & 1, out = pass & 1;  // double-buffer halves
            const PassRows cur = sched[pass - 1];
            const int din = pass > 1 ? sched[pass - 2].rows : 1;  // rows this pass decides
            const int dout = cur.rows > 0 ? cur.rows : 1;         // row slots of its grid
            // the last pass only decides: one wave a request
            const int nseg = pass == 1 ? pl.nseg_first : (cur.rows == 0 ? 1 : pl.nseg);
            PassParams pp{};
            pp.target = a.target;
            pp.x = a.x;
            pp.ell = a.ell;
            pp.qx = a.qx;
            pp.temperature = a.temperature;
            pp.B = a.B;
            pp.gamma = a.gamma;
            pp.V = a.V;
            pp.j0 = cur.j0;
            pp.vec = vec_t;
            pp.nseg = nseg;
            pp.seg_len = pass == 1 ? pl.seg_len_first : pl.seg_len;
            pp.nseg_in = pass == 2 ? pl.nseg_first : pl.nseg;
            pp.seg_stride = pl.nseg_max;
            pp.row_stride = rs;
            pp.key0 = a.key0;
            pp.key1 = a.key1;
            pp.round32 = a.round32;
            pp.off = w.off;
            pp.prep = (pass == 1 && prep_in_kernel) ? 1 : 0;
            pp.n_target_rows = a.n_target_rows;
            pp.row_offsets = a.row_offsets;
            pp.req_flags = w.req_flags;
            pp.resid_out = a.resid_out;
            pp.act_in = w.act + size_t(in) * a.B;
            pp.pm_in = w.seg_m + in * half;
            pp.ps_in = w.seg_s + in * half;
            pp.pv_in = w.seg_v + in * half;
            pp.pi_in = w.seg_i + in * half;
            pp.tx_in = w.seg_tx + size_t(in) * kPassRows * a.B;
            pp.act_out = w.act + size_t(out) * a.B;
            pp.pm_out = w.seg_m + out * half;
            pp.ps_out = w.seg_s + out * half;
            pp.pv_out = w.seg_v + out * half;
            pp.pi_out = w.seg_i + out * half;
            pp.tx_out = w.seg_tx + size_t(out) * kPassRows * a.B;
            pp.mode = w.mode;
            pp.jpos = w.jpos;
            pp.fin_lse2 = w.fin_lse2;
            pp.prev = w.prev;
            pp.erow_mode = a.erow_mode;
            pp.lse2q = w.lse2q;
            pp.anchor = a.anchor;
            pp.lse_q = a.lse_q;
            pp.n_accept_out = a.n_accept_out;
            pp.tokens_out = a.tokens_out;
            pp.diag_out = a.diag_out;
            pp.tail_cnt = tail_from ? w.tail_cnt : nullptr;
            static const char *const names[] = {"verify_pass1", "verify_pass2", "verify_pass3", "verify_pass4",
                                                "verify_pass5", "verify_pass6", "verify_pass7", "verify_pass8+"};
            const dim3 grid(size_t((a.B + 3) / 4) * nseg * dout);
            const char *name = names[std::min(pass, 8) - 1];
            if (pass == 1 && dout == 1)
                launch_kernel(name, (verify_pass_kernel<true, 1, 1>), grid, dim3(256), s, pp);
            else if (pass == 1)
                launch_kernel(name, (verify_pass_kernel<true, 1, 2>), grid, dim3(256), s, pp);
            else if (din == 1 && dout == 1)
                launch_kernel(name, (verify_pass_kernel<false, 1, 1>), grid, dim3(256), s, pp);
            else if (din == 1)
                launch_kernel(name, (verify_pass_kernel<false, 1, 2>), grid, dim3(256), s, pp);
            else if (dout == 1)
                launch_kernel(name, (verify_pass_kernel<false, 2, 1>), grid, dim3(256), s, pp);
            else
                launch_kernel(name, (verify_pass_kernel<false, 2, 2>), grid, dim3(256), s, pp);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (tail_from) {
            const int last = npass & 1;  // the half the last pass wrote
            WalkParams tp = walk_params();
            tp.tail_from = tail_from;
            tp.tail_din = tail_din;
            tp.nseg_in = npass == 1 ? pl.nseg_first : pl.nseg;
            tp.seg_stride = pl.nseg_max;
            tp.row_stride = rs;
            tp.act_in = w.act + size_t(last) * a.B;
            tp.pm_in = w.seg_m + last * half;
            tp.ps_in = w.seg_s + last * half;
            tp.pv_in = w.seg_v + last * half;
            tp.pi_in = w.seg_i + last * half;
            tp.tx_in = w.seg_tx + size_t(last) * kPassRows * a.B;
            const int nt = a.gamma + 2 - tail_from;
            launch_kernel("verify_tail", verify_tail_kernel, dim3(size_t(a.B) * nt), dim3(kWalkThreads), s, tp);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    {
        DrawParams dp{};
        dp.U = a.U;
        dp.target = a.target;
        dp.W1 = a.W1;
        dp.W2 = a.W2;
        dp.anchor = a.anchor;
        dp.x = a.x;
        dp.lse_q = a.lse_q;
        dp.temperature = a.temperature;
        dp.B = a.B;
        dp.gamma = a.gamma;
        dp.V = a.V;
        dp.nbg = pl.draw_nbg;
        dp.ntiles = pl.tile.ntiles;
        dp.tiles_per_chunk = pl.tile.tiles_per_chunk;
        dp.nchunk = pl.tile.nchunk;
        dp.key0 = a.key0;
        dp.key1 = a.key1;
        dp.round32 = a.round32;
        dp.mode = w.mode;
        dp.jpos = w.jpos;
        dp.off = w.off;
        dp.fin_lse2 = w.fin_lse2;
        dp.prev = w.prev;
        dp.lse2q = w.lse2q;
        dp.dw_sum = w.dw_sum;
        dp.dw_bl = w.dw_bl;
        dp.dw_bt = w.dw_bt;
        const dim3 grid(pl.draw_blocks), block(64 * pl.draw_nw);
        const bool vec = vec_u && vec_t, small = pl.draw_nw == kDrawSmallWaves;
        if (vec && small)
            launch_kernel("verify_draw", (verify_draw_kernel<WT, R, true, kDrawSmallWaves>), grid, block, s, dp);
        else if (small)
            launch_kernel("verify_draw", (verify_draw_kernel<WT, R, false, kDrawSmallWaves>), grid, block, s, dp);
        else if (vec)
            launch_kernel("verify_draw", (verify_draw_kernel<WT, R, true, kDrawThreads / 64>), grid, block, s, dp);
        else
            launch_kernel("verify_draw", (verify_draw_kernel<WT, R, false, kDrawThreads / 64>), grid, block, s, dp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        FinishParams fp{};
        fp.U = a.U;
        fp.target = a.target;
        fp.W1 = a.W1;
        fp.W2 = a.W2;
        fp.anchor = a.anchor;
        fp.x = a.x;
        fp.lse_q = a.lse_q;
        fp.temperature = a.temperature;
        fp.B = a.B;
        fp.gamma = a.gamma;
        fp.V = a.V;
        fp.nchunk = pl.tile.nchunk;
        fp.ntiles = pl.tile.ntiles;
        fp.key0 = a.key0;
        fp.key1 = a.key1;
        fp.round32 = a.round32;
        fp.status = w.status;
        fp.req_flags = w.req_flags;
        fp.mode = w.mode;
        fp.n_accept = a.n_accept_out;
        fp.off = w.off;
        fp.fin_lse2 = w.fin_lse2;
        fp.jpos = w.jpos;
        fp.prev = w.prev;
        fp.lse2q = w.lse2q;
        fp.dw_sum = w.dw_sum;
        fp.dw_bl = w.dw_bl;
        fp.dw_bt = w.dw_bt;
        fp.tokens_out = a.tokens_out;
        fp.out_offsets = a.out_offsets;
        fp.resid_out = a.resid_out;
        launch_kernel("verify_finish", (verify_finish_kernel<WT, R>), dim3((a.B + 3) / 4 + 1), dim3(256), s, fp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

VerifyPlan verify_plan(int B, int gamma, int V) {
    VerifyPlan p{};
    // a workgroup a request (the walk) once the batch fills most of the chip;
    // smaller batches spread each row over many waves (the position passes)
    p.walk = B >= kWalkMinBatch;
    // the walk's last rows in parallel, while the batch leaves CUs idle then
    p.tail_from = (p.walk && B <= kTailMaxBatch && gamma >= kTailMinGamma) ? kTailFrom : 0;
    // Position passes split a row into segments of whole float4 groups: the
    // first pass, which reads every request's row, in a few long ones (long
    // streams per workgroup), the later ones, which read fewer and fewer rows,
    // in up to kSegLater short ones (more waves per row).
    const int n4 = (V + 3) / 4;
    auto split = [&](int k, int &nseg, int &len) {
        len = 4 * ((n4 + k - 1) / k);
        nseg = (V + len - 1) / len;
    };
    split(kSegFirst, p.nseg_first, p.seg_len_first);
    split(kSegLater, p.nseg, p.seg_len);
    p.nseg_max = std::max(p.nseg_first, p.nseg);
    p.nbb = (B + 31) / 32;
    // 8-wave workgroups holding two one-tile stages of W2 rows and wave
    // regions (160 KB of LDS at bf16 rank 256): one a CU, so about 256 of them
    // for the requests; a batch of at most two request blocks: 2-wave ones,
    // two a CU, about 512
    p.draw_nw = p.nbb <= kDrawSmallWaves ? kDrawSmallWaves : kDrawThreads / 64;
    p.tile = tile_walk_plan(B, V, p.draw_nw, p.draw_nw == kDrawSmallWaves ? 512 : 256, 1);
    // the draw list holds every drawing request in B entries
    p.draw_nbg = (p.nbb + p.draw_nw - 1) / p.draw_nw;
    p.draw_blocks = p.tile.nchunk * p.draw_nbg;
    return p;
}

VerifyWork verify_carve(void *ws, int B, int gamma, int V, const VerifyPlan &p, size_t *bytes) {
    (void)V;
    Carve c(ws);
    VerifyWork w{};
    w.status = c.take<int32_t>(4);  // first: dspark_verify_check reads word 0
    w.req_flags = c.take<int32_t>(B);
    w.off = c.take<int32_t>(size_t(B) + 1);
    if (!p.walk) {  // the position passes' double-buffered segment statistics
        w.act = c.take<int32_t>(size_t(2) * B);
        const size_t ns = size_t(2) * kPassRows * B * p.nseg_max;
        w.seg_m = c.take<float>(ns);
        w.seg_s = c.take<float>(ns);
        w.seg_v = c.take<float>(ns);
        w.seg_i = c.take<int32_t>(ns);
        w.seg_tx = c.take<float>(size_t(2) * kPassRows * B);
    }
    if (B <= kTailMaxBatch) {  // the tail kernel's, after the walk or the passes (rows 2 .. gamma + 1 at most)
        const size_t nt = size_t(B) * std::max(gamma, 1);
        w.tail_flag = c.take<int32_t>(B);
        w.tail_cnt = c.take<int32_t>(B);
        w.tail_lse2 = c.take<float>(nt);
        w.tail_tx = c.take<float>(nt);
        w.tail_amax = c.take<int32_t>(nt);
    }
    w.fin_lse2 = c.take<float>(B);
    w.prev = c.take<int32_t>(B);
    w.lse2q = c.take<float>(B);
    w.mode = c.take<int32_t>(B);
    w.jpos = c.take<int32_t>(B);
    const size_t nd = size_t(B) * p.tile.nchunk;
    w.dw_sum = c.take<float>(nd);
    w.dw_bl = c.take<float>(nd);
    w.dw_bt = c.take<int32_t>(nd);
    if (bytes) *bytes = c.off + 256;
    return w;
}

hipError_t launch_verify(const VerifyArgs &a, const VerifyPlan &p, const VerifyWork &w, hipStream_t s) {
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
