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
// for the same rule).  The draw from r (and from p for the bonus token) is
// Gumbel-max over log r(v) with per-vocabulary Philox noise (stream 2).
//
// Kernels, in launch order:
//   verify_prep      1 workgroup: packed row offsets (scan of 1 + ell, or the
//                    caller's, checked), row -> (request, position) map.
//   verify_rowstats  1 workgroup per packed target row: one coalesced pass
//                    for logsumexp(t / T) in base 2, the lowest-index argmax
//                    and t(x_k).
//   verify_accept    1 workgroup: per request the accept tests u*q < p in
//                    order, n = leading accepts, greedy outputs, the output
//                    offsets and the ascending lists of residual and bonus
//                    requests.
//   verify_draw      one wave per (32 listed requests x vocabulary chunk):
//                    residual rows recompute q_j with the draft's MFMA bias
//                    tile and form max(p_j - q_j, 0); bonus rows use p; both
//                    keep the Gumbel-perturbed best score per chunk.
//   verify_finish    one wave per drawing request: merges the chunk partials
//                    into the emitted token and the residual mass S.
#include "device_common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace dspark {

namespace {

constexpr int kStatusBadEll = 1;
constexpr int kStatusBadOffsets = 2;
constexpr int kStatusRowsOutOfRange = 4;

constexpr int kModeDone = 0;
constexpr int kModeResidual = 1;
constexpr int kModeBonus = 2;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
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
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) argmax_merge(v, i, __shfl_xor(v, o), __shfl_xor(i, o));
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
    int B, gamma, rows_max, n_target_rows;
    int32_t *status, *off, *row_req, *row_pos, *mode;
};

__global__ __launch_bounds__(1024) void verify_prep_kernel(PrepParams p) {
    __shared__ int lds[1024];
    const int t = threadIdx.x;
    const int seg = (p.B + 1023) / 1024;
    const int b0 = min(p.B, t * seg), b1 = min(p.B, b0 + seg);
    for (int i = t; i < p.rows_max; i += 1024) {
        p.row_req[i] = -1;
        p.row_pos[i] = 0;
    }
    int flags = 0;
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        int e = p.ell[b];
        if (e < 0 || e > p.gamma) {
            flags |= kStatusBadEll;
            e = min(max(e, 0), p.gamma);
        }
        local += 1 + e;
    }
    int total = 0;
    int base = block_exclusive_scan<1024>(local, lds, &total);
    // offsets: computed, or the caller's after a consistency check
    for (int b = b0; b < b1; ++b) {
        const int e_raw = p.ell[b];
        const int e = min(max(e_raw, 0), p.gamma);
        int o = base;
        bool ok = (e_raw == e);
        if (p.row_offsets) {
            o = p.row_offsets[b];
            const int o1 = p.row_offsets[b + 1];
            if (o < 0 || o1 - o != 1 + e_raw) {
                ok = false;
                flags |= kStatusBadOffsets;
            }
        }
        if (ok && (o + e + 1 > p.n_target_rows || o + e + 1 > p.rows_max)) {
            ok = false;
            flags |= kStatusRowsOutOfRange;
        }
        p.off[b] = ok ? o : 0;
        p.mode[b] = ok ? kModeDone : -1;
        base += 1 + e;
    }
    if (t == 1023) p.off[p.B] = p.row_offsets ? p.row_offsets[p.B] : total;
    // status flags: OR across the group
    lds[t] = flags;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if (t < o) lds[t] |= lds[t + o];
        __syncthreads();
    }
    if (t == 0) {
        p.status[0] = lds[0];
        p.status[1] = min(p.rows_max, p.row_offsets ? max(0, p.row_offsets[p.B]) : total);
        p.status[2] = 0;
        p.status[3] = 0;
    }
    __syncthreads();  // every row_req entry is initialised before the fill below
    for (int b = b0; b < b1; ++b) {
        if (p.mode[b] < 0) continue;
        const int e = p.ell[b];
        const int o = p.off[b];
        for (int i = 0; i <= e; ++i) {
            p.row_req[o + i] = b;
            p.row_pos[o + i] = i + 1;
        }
    }
}

// ------------------------------------------------------------------ rowstats

struct RowStatsParams {
    const float *target;
    const int32_t *x, *ell;
    const float *temperature;
    int V, gamma, nrchunk, vec;
    const int32_t *status, *row_req, *row_pos;
    float *row_lse2, *row_tx2;
    int32_t *row_amax;
};

__global__ __launch_bounds__(256) void verify_rowstats_kernel(RowStatsParams p) {
    const int row = blockIdx.x;
    if (row >= p.status[1]) return;
    const int req = p.row_req[row];
    if (req < 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float T = p.temperature[req];
    const float sc = T > 0.f ? kLog2e / T : 1.0f;
    const float *trow = p.target + size_t(row) * p.V;
    const bool vec = p.vec != 0;
    float rm = kNegInf, rs = 0.f, av = kNegInf;
    int ai = 0x7fffffff;
    for (int c = wave; c < p.nrchunk; c += 4) {
        const int cb = c * kRowChunk;
        float vals[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 t4 = load4_masked(trow, cb + 4 * (lane + 64 * q), p.V, vec);
            vals[4 * q + 0] = t4.x * sc;
            vals[4 * q + 1] = t4.y * sc;
            vals[4 * q + 2] = t4.z * sc;
            vals[4 * q + 3] = t4.w * sc;
        }
        float m = vals[0];
        float bv = vals[0];
        int bi = cb + 4 * lane;
#pragma unroll
        for (int e = 1; e < 32; ++e) {
            m = fmaxf(m, vals[e]);
            if (vals[e] > bv) {
                bv = vals[e];
                bi = cb + 4 * (lane + 64 * (e >> 2)) + (e & 3);
            }
        }
        m = wave_max(m);
        const float ms = (m == kNegInf) ? 0.f : m;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) s += fast_exp2(vals[e] - ms);
        s = wave_sum(s);
        wave_argmax(bv, bi);
        lse_merge(rm, rs, m, s);
        argmax_merge(av, ai, bv, bi);
    }
    __shared__ float sm[4], ss[4], sv[4];
    __shared__ int si[4];
    if (lane == 0) {
        sm[wave] = rm;
        ss[wave] = rs;
        sv[wave] = av;
        si[wave] = ai;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = sm[0], s = ss[0], v = sv[0];
        int i = si[0];
        for (int w = 1; w < 4; ++w) {
            lse_merge(m, s, sm[w], ss[w]);
            argmax_merge(v, i, sv[w], si[w]);
        }
        p.row_lse2[row] = (m == kNegInf) ? kNegInf : m + fast_log2(s);
        p.row_amax[row] = min(max(i, 0), p.V - 1);
        const int pos = p.row_pos[row];
        if (pos <= p.ell[req]) {
            int xk = p.x[size_t(req) * p.gamma + pos - 1];
            xk = min(max(xk, 0), p.V - 1);
            p.row_tx2[row] = trow[xk] * sc;
        } else {
            p.row_tx2[row] = kNegInf;
        }
    }
}

// ------------------------------------------------------------------ accept

struct AcceptParams {
    const int32_t *ell, *x;
    const float *qx, *temperature;
    int B, gamma;
    uint32_t key0, key1, round32;
    int32_t *status;
    const int32_t *off;
    const float *row_lse2, *row_tx2;
    const int32_t *row_amax;
    int32_t *mode, *jpos, *resid_list, *bonus_list;
    int32_t *n_accept_out, *tokens_out, *out_offsets;
    float *diag_out, *resid_out;
};

__global__ __launch_bounds__(1024) void verify_accept_kernel(AcceptParams p) {
    __shared__ int lds[1024];
    const int t = threadIdx.x;
    const int seg = (p.B + 1023) / 1024;
    const int b0 = min(p.B, t * seg), b1 = min(p.B, b0 + seg);
    const float nan = __builtin_nanf("");
    int emitted = 0, nres = 0, nbon = 0;
    for (int b = b0; b < b1; ++b) {
        int32_t *tok = p.tokens_out + size_t(b) * (p.gamma + 1);
        for (int i = 0; i <= p.gamma; ++i) tok[i] = -1;
        if (p.diag_out)
            for (int i = 0; i < 2 * (p.gamma + 1); ++i) p.diag_out[size_t(b) * 2 * (p.gamma + 1) + i] = nan;
        if (p.resid_out) p.resid_out[b] = -1.f;
        if (p.mode[b] < 0) {
            p.n_accept_out[b] = -1;
            continue;
        }
        const int L = p.ell[b];
        const int o = p.off[b];
        const bool sampled = p.temperature[b] > 0.f;
        int n = 0;
        bool rejected = false;
        for (int k = 1; k <= L; ++k) {
            const int row = o + k - 1;
            const int xk = p.x[size_t(b) * p.gamma + k - 1];
            bool acc;
            float pk, ratio;
            if (sampled) {
                pk = fast_exp2(p.row_tx2[row] - p.row_lse2[row]);
                const float qk = p.qx[size_t(b) * p.gamma + k - 1];
                const float u =
                    uniform01(scalar_word(kStreamAccept, k, uint32_t(b), p.round32, p.key0, p.key1));
                acc = u * qk < pk;
                ratio = qk > 0.f ? fminf(1.f, pk / qk) : 1.f;
            } else {
                acc = (xk == p.row_amax[row]);
                pk = acc ? 1.f : 0.f;
                ratio = pk;
            }
            if (p.diag_out) {
                p.diag_out[(size_t(b) * (p.gamma + 1) + (k - 1)) * 2 + 0] = pk;
                p.diag_out[(size_t(b) * (p.gamma + 1) + (k - 1)) * 2 + 1] = ratio;
            }
            if (!acc) {
                rejected = true;
                break;
            }
            tok[k - 1] = xk;
            n = k;
        }
        p.n_accept_out[b] = n;
        p.jpos[b] = n + 1;
        emitted += n + 1;
        if (!sampled) {
            tok[n] = p.row_amax[o + n];
            p.mode[b] = kModeDone;
        } else if (rejected) {
            p.mode[b] = kModeResidual;
            ++nres;
        } else {
            p.mode[b] = kModeBonus;
            ++nbon;
        }
    }
    int tot_emit = 0, tot_res = 0, tot_bon = 0;
    const int base_emit = block_exclusive_scan<1024>(emitted, lds, &tot_emit);
    const int base_res = block_exclusive_scan<1024>(nres, lds, &tot_res);
    const int base_bon = block_exclusive_scan<1024>(nbon, lds, &tot_bon);
    int e = base_emit, r = base_res, q = base_bon;
    for (int b = b0; b < b1; ++b) {
        if (p.out_offsets) p.out_offsets[b] = e;
        if (p.mode[b] >= 0) e += p.n_accept_out[b] + 1;
        if (p.mode[b] == kModeResidual) p.resid_list[r++] = b;
        if (p.mode[b] == kModeBonus) p.bonus_list[q++] = b;
    }
    if (t == 0) {
        if (p.out_offsets) p.out_offsets[p.B] = tot_emit;
        p.status[2] = tot_res;
        p.status[3] = tot_bon;
    }
}

// ------------------------------------------------------------------ draw

struct DrawParams {
    const float *U, *target;
    const void *W1, *W2;
    const int32_t *anchor, *x;
    const float *lse_q, *temperature;
    int B, gamma, V;
    int tiles_per_chunk, nchunk;
    int vec_u, vec_t;
    uint32_t key0, key1, round32;
    const int32_t *status, *resid_list, *bonus_list, *jpos, *off;
    const float *row_lse2;
    float *dw_sum, *dw_br, *dw_bp;
    int32_t *dw_ir, *dw_ip;
};

template <typename WT, int R>
__global__ __launch_bounds__(256) void verify_draw_kernel(DrawParams p) {
    const int nres = p.status[2], nbon = p.status[3];
    const int nblk_r = (nres + 31) / 32, nblk = nblk_r + (nbon + 31) / 32;
    const int lane = threadIdx.x & 63;
    const int gw = xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
    if (gw >= nblk * p.nchunk) return;
    const int lb = gw % nblk;
    const int chunk = gw / nblk;
    const bool resid_blk = lb < nblk_r;  // uniform across the wave
    const int n = lane & 31, h = lane >> 5;
    int e, req, slot;
    bool ok;
    if (resid_blk) {
        e = lb * 32 + n;
        ok = e < nres;
        req = p.resid_list[ok ? e : nres - 1];
        slot = e;
    } else {
        e = (lb - nblk_r) * 32 + n;
        ok = e < nbon;
        req = p.bonus_list[ok ? e : nbon - 1];
        slot = p.B + e;
    }
    const int j = p.jpos[req];
    const float sc = kLog2e / p.temperature[req];
    const int trow_i = p.off[req] + j - 1;
    const float *trow = p.target + size_t(trow_i) * p.V;
    const float lse2t = p.row_lse2[trow_i];
    const bool vec_t = p.vec_t != 0, vec_u = p.vec_u != 0;

    const WT *W2 = static_cast<const WT *>(p.W2);
    EFrags<WT, R> ef;
    const float *urow = p.U;
    float lse2q = 0.f;
    if (resid_blk) {
        int prev = (j == 1) ? p.anchor[req] : p.x[size_t(req) * p.gamma + j - 2];
        prev = min(max(prev, 0), p.V - 1);
        ef.load(static_cast<const WT *>(p.W1) + size_t(prev) * R, h);
        urow = p.U + (size_t(req) * p.gamma + j - 1) * p.V;
        lse2q = p.lse_q[size_t(req) * p.gamma + j - 1] * kLog2e;
    }

    const int v_begin = chunk * p.tiles_per_chunk * 32;
    const int v_end = min(p.V, v_begin + p.tiles_per_chunk * 32);
    float S = 0.f, br = kNegInf, bp = kNegInf;
    int ir = v_begin + 4 * h, ip = v_begin + 4 * h;
    for (int v0 = v_begin; v0 < v_end; v0 += 32) {
        f32x16_t acc = {};
        if (resid_blk) {
            const int vrow = min(v0 + n, p.V - 1);
            acc = bias_tile(ef, W2 + size_t(vrow) * R, h);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int vb = v0 + 8 * i + 4 * h;
            const float4 t4 = load4_masked(trow, vb, p.V, vec_t);
            float4 u4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (resid_blk) u4 = load4_masked(urow, vb, p.V, vec_u);
            const uint4 w = noise_block(kStreamResample, j, uint32_t(vb >> 2), uint32_t(req), p.round32, p.key0,
                                        p.key1);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float tt = f4get(t4, jj) * sc;  // log2 p + lse2t
                const float g = gumbel2(u4get(w, jj));
                const float sp = tt + g;
                if (sp > bp) {
                    bp = sp;
                    ip = vb + jj;
                }
                if (resid_blk) {
                    const float z2 = (f4get(u4, jj) + acc[4 * i + jj]) * sc;
                    const float q = fast_exp2(z2 - lse2q);
                    const float pp = fast_exp2(tt - lse2t);
                    const float res = fmaxf(pp - q, 0.f);
                    S += res;
                    const float sr = res > 0.f ? fast_log2(res) + g : kNegInf;
                    if (sr > br) {
                        br = sr;
                        ir = vb + jj;
                    }
                }
            }
        }
    }
    // merge the two lane halves that share a request
    S += __shfl_xor(S, 32);
    argmax_merge(br, ir, __shfl_xor(br, 32), __shfl_xor(ir, 32));
    argmax_merge(bp, ip, __shfl_xor(bp, 32), __shfl_xor(ip, 32));
    if (h == 0 && ok) {
        const size_t o = size_t(slot) * p.nchunk + chunk;
        p.dw_sum[o] = S;
        p.dw_br[o] = br;
        p.dw_ir[o] = ir;
        p.dw_bp[o] = bp;
        p.dw_ip[o] = ip;
    }
}

// ------------------------------------------------------------------ finish

struct FinishParams {
    int B, gamma, V, nchunk;
    const int32_t *status, *mode, *n_accept, *resid_list, *bonus_list;
    const float *dw_sum, *dw_br, *dw_bp;
    const int32_t *dw_ir, *dw_ip;
    int32_t *tokens_out;
    float *resid_out;
};

__device__ int list_position(const int32_t *list, int n, int b) {
    int lo = 0, hi = n - 1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int v = list[mid];
        if (v == b) return mid;
        if (v < b) lo = mid + 1;
        else hi = mid - 1;
    }
    return 0;
}

__global__ __launch_bounds__(256) void verify_finish_kernel(FinishParams p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= p.B) return;
    const int mode = p.mode[b];
    if (mode != kModeResidual && mode != kModeBonus) return;
    const int slot = (mode == kModeResidual) ? list_position(p.resid_list, p.status[2], b)
                                             : p.B + list_position(p.bonus_list, p.status[3], b);
    float S = 0.f, br = kNegInf, bp = kNegInf;
    int ir = 0x7fffffff, ip = 0x7fffffff;
    for (int c = lane; c < p.nchunk; c += 64) {
        const size_t o = size_t(slot) * p.nchunk + c;
        S += p.dw_sum[o];
        argmax_merge(br, ir, p.dw_br[o], p.dw_ir[o]);
        argmax_merge(bp, ip, p.dw_bp[o], p.dw_ip[o]);
    }
    S = wave_sum(S);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        argmax_merge(br, ir, __shfl_xor(br, o), __shfl_xor(ir, o));
        argmax_merge(bp, ip, __shfl_xor(bp, o), __shfl_xor(ip, o));
    }
    if (lane == 0) {
        // a residual with no mass left (p = q to rounding) falls back to p_j
        const bool use_res = mode == kModeResidual && S > 0.f && br > kNegInf;
        const int y = min(max(use_res ? ir : ip, 0), p.V - 1);
        p.tokens_out[size_t(b) * (p.gamma + 1) + p.n_accept[b]] = y;
        if (p.resid_out && mode == kModeResidual) p.resid_out[b] = S;
    }
}

template <typename WT, int R>
hipError_t launch_typed(const VerifyArgs &a, const VerifyPlan &pl, const VerifyWork &w, hipStream_t s) {
    hipError_t e;
    {
        PrepParams pp{a.ell, a.row_offsets, a.B, a.gamma, pl.rows_max, a.n_target_rows,
                      w.status, w.off, w.row_req, w.row_pos, w.mode};
        int t = prof_begin("verify_prep", s);
        hipLaunchKernelGGL(verify_prep_kernel, dim3(1), dim3(1024), 0, s, pp);
        prof_end(t, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool vec_t = (reinterpret_cast<uintptr_t>(a.target) % 16 == 0) && (a.V % 4 == 0);
    const bool vec_u = (reinterpret_cast<uintptr_t>(a.U) % 16 == 0) && (a.V % 4 == 0);
    {
        RowStatsParams rp{a.target, a.x, a.ell, a.temperature, a.V, a.gamma, pl.nrchunk, vec_t,
                          w.status, w.row_req, w.row_pos, w.row_lse2, w.row_tx2, w.row_amax};
        int t = prof_begin("verify_rowstats", s);
        hipLaunchKernelGGL(verify_rowstats_kernel, dim3(pl.rows_max), dim3(256), 0, s, rp);
        prof_end(t, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        AcceptParams ap{a.ell, a.x, a.qx, a.temperature, a.B, a.gamma, a.key0, a.key1, a.round32,
                        w.status, w.off, w.row_lse2, w.row_tx2, w.row_amax, w.mode, w.jpos, w.resid_list,
                        w.bonus_list, a.n_accept_out, a.tokens_out, a.out_offsets, a.diag_out, a.resid_out};
        int t = prof_begin("verify_accept", s);
        hipLaunchKernelGGL(verify_accept_kernel, dim3(1), dim3(1024), 0, s, ap);
        prof_end(t, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
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
        dp.tiles_per_chunk = pl.tile.tiles_per_chunk;
        dp.nchunk = pl.tile.nchunk;
        dp.vec_u = vec_u;
        dp.vec_t = vec_t;
        dp.key0 = a.key0;
        dp.key1 = a.key1;
        dp.round32 = a.round32;
        dp.status = w.status;
        dp.resid_list = w.resid_list;
        dp.bonus_list = w.bonus_list;
        dp.jpos = w.jpos;
        dp.off = w.off;
        dp.row_lse2 = w.row_lse2;
        dp.dw_sum = w.dw_sum;
        dp.dw_br = w.dw_br;
        dp.dw_bp = w.dw_bp;
        dp.dw_ir = w.dw_ir;
        dp.dw_ip = w.dw_ip;
        int t = prof_begin("verify_draw", s);
        hipLaunchKernelGGL((verify_draw_kernel<WT, R>), dim3(pl.draw_blocks), dim3(256), 0, s, dp);
        prof_end(t, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        FinishParams fp{a.B, a.gamma, a.V, pl.tile.nchunk, w.status, w.mode, a.n_accept_out, w.resid_list,
                        w.bonus_list, w.dw_sum, w.dw_br, w.dw_bp, w.dw_ir, w.dw_ip, a.tokens_out, a.resid_out};
        int t = prof_begin("verify_finish", s);
        hipLaunchKernelGGL(verify_finish_kernel, dim3((a.B + 3) / 4), dim3(256), 0, s, fp);
        prof_end(t, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

VerifyPlan verify_plan(int B, int gamma, int V) {
    VerifyPlan p{};
    p.rows_max = B * (gamma + 1);
    p.nrchunk = (V + kRowChunk - 1) / kRowChunk;
    p.nbb = (B + 31) / 32;
    p.tile = draft_plan(B, V);
    // the residual and bonus lists hold at most B requests but each rounds up to 32
    p.draw_blocks = ((p.nbb + 1) * p.tile.nchunk + 3) / 4;
    return p;
}

VerifyWork verify_carve(void *ws, int B, int gamma, int V, const VerifyPlan &p, size_t *bytes) {
    (void)gamma;
    (void)V;
    Carve c(ws);
    VerifyWork w{};
    w.status = c.take<int32_t>(4);
    w.off = c.take<int32_t>(size_t(B) + 1);
    w.row_req = c.take<int32_t>(p.rows_max);
    w.row_pos = c.take<int32_t>(p.rows_max);
    w.row_lse2 = c.take<float>(p.rows_max);
    w.row_amax = c.take<int32_t>(p.rows_max);
    w.row_tx2 = c.take<float>(p.rows_max);
    w.mode = c.take<int32_t>(B);
    w.jpos = c.take<int32_t>(B);
    w.resid_list = c.take<int32_t>(B);
    w.bonus_list = c.take<int32_t>(B);
    const size_t nd = size_t(2) * B * p.tile.nchunk;
    w.dw_sum = c.take<float>(nd);
    w.dw_br = c.take<float>(nd);
    w.dw_bp = c.take<float>(nd);
    w.dw_ir = c.take<int32_t>(nd);
    w.dw_ip = c.take<int32_t>(nd);
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
