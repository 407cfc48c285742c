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
//   verify_prep      1 workgroup: packed row offsets (scan of 1 + ell, or the
//                    caller's, checked), row -> (request, position) map.
//   verify_rowstats  1 workgroup per packed target row: one coalesced
//                    streaming pass for logsumexp(t / T) in base 2, the
//                    lowest-index argmax and t(x_k).
//   verify_accept    1 workgroup: per request the accept tests u*q < p in
//                    order, n = leading accepts, greedy outputs, the output
//                    offsets and the ascending lists of residual and bonus
//                    requests.
//   verify_draw      level 1: waves of 32 listed requests walk vocabulary
//                    chunks; residual rows recompute q_j with the draft's
//                    LDS-staged MFMA bias tile and sum max(p_j - q_j, 0) per
//                    tile, bonus rows take tile logsumexps of p; the tiles
//                    race with their noise.
//   verify_finish    level 2: one wave per drawing request merges the chunk
//                    partials, recomputes the winning tile's 32 entries and
//                    races them; writes the emitted token and S.
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
    int V, gamma, vec;
    const int32_t *status, *row_req, *row_pos;
    float *row_lse2, *row_tx2;
    int32_t *row_amax;
};

// One workgroup streams one packed target row: every thread keeps its own
// running max / sum of exp2 (base 2) and argmax over batches of eight float4
// loads, and the workgroup merges the 256 states at the end.
__global__ __launch_bounds__(256) void verify_rowstats_kernel(RowStatsParams p) {
    const int row = blockIdx.x;
    if (row >= p.status[1]) return;
    const int req = p.row_req[row];
    if (req < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float T = p.temperature[req];
    const float sc = T > 0.f ? kLog2e / T : 1.0f;
    const float *trow = p.target + size_t(row) * p.V;
    float m = kNegInf, s = 0.f, av = kNegInf;
    int ai = 0x7fffffff;
    if (p.vec) {
        const float4 *r4 = reinterpret_cast<const float4 *>(trow);
        const int nq = p.V >> 2;
        constexpr int U = 8;
        for (int q0 = tid; q0 < nq; q0 += 256 * U) {
            float4 xs[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = q0 + 256 * u;
                xs[u] = q < nq ? r4[q] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
            }
            float bm = kNegInf;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xs[u].x *= sc;
                xs[u].y *= sc;
                xs[u].z *= sc;
                xs[u].w *= sc;
                bm = fmaxf(fmaxf(bm, fmaxf(xs[u].x, xs[u].y)), fmaxf(xs[u].z, xs[u].w));
            }
            const float mn = fmaxf(m, bm);
            if (mn != kNegInf) {
                float add = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    add += fast_exp2(xs[u].x - mn) + fast_exp2(xs[u].y - mn) + fast_exp2(xs[u].z - mn) +
                           fast_exp2(xs[u].w - mn);
                s = s * fast_exp2(m - mn) + add;
                m = mn;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = 4 * (q0 + 256 * u);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float xv = f4get(xs[u], j);
                    if (xv > av) {
                        av = xv;
                        ai = v + j;
                    }
                }
            }
        }
    } else {
        for (int v = tid; v < p.V; v += 256) {
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
    // merge the 256 thread states: within the wave, then across the 4 waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lse_merge(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
        argmax_merge(av, ai, __shfl_xor(av, o), __shfl_xor(ai, o));
    }
    __shared__ float sm[4], ss[4], sv[4];
    __shared__ int si[4];
    if (lane == 0) {
        sm[wave] = m;
        ss[wave] = s;
        sv[wave] = av;
        si[wave] = ai;
    }
    __syncthreads();
    if (tid == 0) {
        float mm = sm[0], s2 = ss[0], v2 = sv[0];
        int i2 = si[0];
        for (int w = 1; w < 4; ++w) {
            lse_merge(mm, s2, sm[w], ss[w]);
            argmax_merge(v2, i2, sv[w], si[w]);
        }
        p.row_lse2[row] = (mm == kNegInf) ? kNegInf : mm + fast_log2(s2);
        p.row_amax[row] = min(max(i2, 0), p.V - 1);
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
    int nw, nbg, ntiles, tiles_per_chunk, nchunk;
    int vec_u, vec_t;
    uint32_t key0, key1, round32;
    const int32_t *status, *resid_list, *bonus_list, *jpos, *off;
    const float *row_lse2;
    float *dw_sum, *dw_bl;
    int32_t *dw_bt;
};

// Level 1 of the resample / bonus draws.  A workgroup of up to 4 waves walks
// the tiles of one vocabulary chunk; each wave holds 32 listed requests.
// Residual waves recompute q_j from the W2 tile (staged in LDS as in the
// draft) and sum max(p_j - q_j, 0) per tile; bonus waves take the tile
// logsumexp of p.  Either way the tile enters a Gumbel race (stream 4).
template <typename WT, int R>
__global__ __launch_bounds__(256) void verify_draw_kernel(DrawParams p) {
    using L = TileLDS<WT, R>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::BYTES];
    const int nres = p.status[2], nbon = p.status[3];
    const int nblk_r = (nres + 31) / 32, nblk = nblk_r + (nbon + 31) / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nthreads = p.nw * 64;
    const int lg = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = lg / p.nbg, bg = lg % p.nbg;
    const int lb0 = bg * p.nw;
    if (lb0 >= nblk) return;                   // the whole workgroup is idle
    const bool need_tiles = lb0 < nblk_r;      // uniform across the workgroup
    const int lb = lb0 + wave;
    const bool wave_ok = lb < nblk;            // uniform across the wave
    const bool resid = lb < nblk_r;            // uniform across the wave
    const int n = lane & 31, h = lane >> 5;
    int e = 0, req = 0, slot = 0;
    bool ok = false;
    if (resid) {
        e = lb * 32 + n;
        ok = e < nres;
        req = p.resid_list[ok ? e : nres - 1];
        slot = e;
    } else if (wave_ok) {
        e = (lb - nblk_r) * 32 + n;
        ok = e < nbon;
        req = p.bonus_list[ok ? e : nbon - 1];
        slot = p.B + e;
    }
    const int j = wave_ok ? p.jpos[req] : 1;
    const float sc = wave_ok ? kLog2e / p.temperature[req] : 1.0f;
    const int trow_i = wave_ok ? p.off[req] + j - 1 : 0;
    const float *trow = p.target + size_t(trow_i) * p.V;
    const float lse2t = wave_ok ? p.row_lse2[trow_i] : 0.f;
    const bool vec_t = p.vec_t != 0, vec_u = p.vec_u != 0;

    const WT *W2 = static_cast<const WT *>(p.W2);
    EFrags<WT, R> ef;
    const float *urow = p.U;
    float lse2q = 0.f;
    if (resid) {
        int prev = (j == 1) ? p.anchor[req] : p.x[size_t(req) * p.gamma + j - 2];
        prev = min(max(prev, 0), p.V - 1);
        ef.load(static_cast<const WT *>(p.W1) + size_t(prev) * R, h);
        urow = p.U + (size_t(req) * p.gamma + j - 1) * p.V;
        lse2q = p.lse_q[size_t(req) * p.gamma + j - 1] * kLog2e;
    }

    const int t_begin = chunk * p.tiles_per_chunk;
    const int t_end = min(p.ntiles, t_begin + p.tiles_per_chunk);
    float S = 0.f, best = kNegInf;
    int bt = t_begin;
    uint4 tw = make_uint4(0u, 0u, 0u, 0u);
    if (need_tiles) tile_issue<WT, R>(W2, t_begin * kTile, p.V, lds, nthreads);
    float4 tcur[4], ucur[4];
    if (wave_ok) load_tile_row(trow, t_begin, h, p.V, vec_t, tcur);
    if (resid) load_tile_row(urow, t_begin, h, p.V, vec_u, ucur);
    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        __builtin_amdgcn_s_waitcnt(0);
        if (need_tiles) __syncthreads();
        const bool more = t + 1 < t_end;
        float4 tnext[4], unext[4];
        if (more) {
            if (need_tiles) tile_issue<WT, R>(W2, (t + 1) * kTile, p.V, lds + (buf ^ 1) * L::BYTES, nthreads);
            if (wave_ok) load_tile_row(trow, t + 1, h, p.V, vec_t, tnext);
            if (resid) load_tile_row(urow, t + 1, h, p.V, vec_u, unext);
        }
        if (wave_ok) {
            if (t == t_begin || (t & 3) == 0)
                tw = noise_block(kStreamResampleTile, j, uint32_t(t) >> 2, uint32_t(req), p.round32, p.key0, p.key1);
            const float g = gumbel2(u4get(tw, t & 3));
            float Lt;
            if (resid) {
                const f32x16_t acc = bias_tile_lds(ef, lds + buf * L::BYTES, lane);
                float sh = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float q = fast_exp2(__builtin_fmaf(f4get(ucur[i], jj) + acc[4 * i + jj], sc, -lse2q));
                        const float pv = fast_exp2(__builtin_fmaf(f4get(tcur[i], jj), sc, -lse2t));
                        sh += fmaxf(pv - q, 0.f);
                    }
                const float st = sh + __shfl_xor(sh, 32);
                S += st;
                Lt = st > 0.f ? fast_log2(st) + g : kNegInf;
            } else {
                float tv[16];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) tv[4 * i + jj] = f4get(tcur[i], jj) * sc;
                float mh = tv[0];
#pragma unroll
                for (int q = 1; q < 16; ++q) mh = fmaxf(mh, tv[q]);
                const float mhs = (mh == kNegInf) ? 0.f : mh;
                float sh = 0.f;
#pragma unroll
                for (int q = 0; q < 16; ++q) sh += fast_exp2(tv[q] - mhs);
                const float mo = __shfl_xor(mh, 32), so = __shfl_xor(sh, 32);
                const float mt = fmaxf(mh, mo);
                const float mts = (mt == kNegInf) ? 0.f : mt;
                const float st = sh * fast_exp2(mh - mts) + so * fast_exp2(mo - mts);
                Lt = mt + fast_log2(st) + g;
            }
            if (Lt > best) {
                best = Lt;
                bt = t;
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tcur[i] = tnext[i];
                ucur[i] = unext[i];
            }
        }
    }
    if (h == 0 && ok) {
        const size_t o = size_t(slot) * p.nchunk + chunk;
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
    const int32_t *status, *mode, *n_accept, *resid_list, *bonus_list, *off;
    const float *row_lse2;
    const float *dw_sum, *dw_bl;
    const int32_t *dw_bt;
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

// Winner of an entry race held by the 32 lower lanes of the wave.
__device__ __forceinline__ int wave_race(float score, int v) {
    float s = (threadIdx.x & 32) ? kNegInf : score;
    int i = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) argmax_merge(s, i, __shfl_xor(s, o), __shfl_xor(i, o));
    return i;
}

// Level 2 of the draws, and the emitted token: one wave per drawing request.
template <typename WT, int R>
__global__ __launch_bounds__(256) void verify_finish_kernel(FinishParams p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= p.B) return;
    const int mode = p.mode[b];
    if (mode != kModeResidual && mode != kModeBonus) return;
    const int slot = (mode == kModeResidual) ? list_position(p.resid_list, p.status[2], b)
                                             : p.B + list_position(p.bonus_list, p.status[3], b);
    float S = 0.f, bl = kNegInf;
    int tile = 0x7fffffff;
    for (int c = lane; c < p.nchunk; c += 64) {
        const size_t o = size_t(slot) * p.nchunk + c;
        S += p.dw_sum[o];
        argmax_merge(bl, tile, p.dw_bl[o], p.dw_bt[o]);
    }
    S = wave_sum(S);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) argmax_merge(bl, tile, __shfl_xor(bl, o), __shfl_xor(tile, o));

    const int j = p.n_accept[b] + 1;
    const float sc = kLog2e / p.temperature[b];
    const int trow_i = p.off[b] + j - 1;
    const float *trow = p.target + size_t(trow_i) * p.V;
    const float lse2t = p.row_lse2[trow_i];
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
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) argmax_merge(b1, t1, __shfl_xor(b1, o), __shfl_xor(t1, o));
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
        int prev = (j == 1) ? p.anchor[b] : p.x[size_t(b) * p.gamma + j - 2];
        prev = min(max(prev, 0), p.V - 1);
        const WT *W1 = static_cast<const WT *>(p.W1);
        const WT *W2 = static_cast<const WT *>(p.W2);
        const float d = bias_entry<WT, R>(W1 + size_t(prev) * R, W2 + size_t(vc) * R, h);
        const float lse2q = p.lse_q[size_t(b) * p.gamma + j - 1] * kLog2e;
        const float logit = p.U[(size_t(b) * p.gamma + j - 1) * p.V + vc] + d;
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
        RowStatsParams rp{a.target, a.x, a.ell, a.temperature, a.V, a.gamma, vec_t,
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
        dp.nw = pl.tile.nw;
        dp.nbg = pl.draw_nbg;
        dp.ntiles = pl.tile.ntiles;
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
        dp.dw_bl = w.dw_bl;
        dp.dw_bt = w.dw_bt;
        int t = prof_begin("verify_draw", s);
        hipLaunchKernelGGL((verify_draw_kernel<WT, R>), dim3(pl.draw_blocks), dim3(64 * pl.tile.nw), 0, s, dp);
        prof_end(t, s);
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
        fp.mode = w.mode;
        fp.n_accept = a.n_accept_out;
        fp.resid_list = w.resid_list;
        fp.bonus_list = w.bonus_list;
        fp.off = w.off;
        fp.row_lse2 = w.row_lse2;
        fp.dw_sum = w.dw_sum;
        fp.dw_bl = w.dw_bl;
        fp.dw_bt = w.dw_bt;
        fp.tokens_out = a.tokens_out;
        fp.resid_out = a.resid_out;
        int t = prof_begin("verify_finish", s);
        hipLaunchKernelGGL((verify_finish_kernel<WT, R>), dim3((a.B + 3) / 4), dim3(256), 0, s, fp);
        prof_end(t, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

VerifyPlan verify_plan(int B, int gamma, int V) {
    VerifyPlan p{};
    p.rows_max = B * (gamma + 1);
    p.nbb = (B + 31) / 32;
    // about 2048 waves of up to 4 over the 1024 SIMDs; chunks of a multiple of
    // 4 tiles share the tile-noise Philox blocks
    const long long nbb = (B + 31) / 32, nw = std::min<long long>(4, nbb);
    p.tile = tile_walk_plan(B, V, 4, std::max<long long>(1, 2048 / nw), 4);
    // the residual and bonus lists hold at most B requests but each rounds up to 32
    p.draw_nbg = (p.nbb + 1 + p.tile.nw - 1) / p.tile.nw;
    p.draw_blocks = p.tile.nchunk * p.draw_nbg;
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
