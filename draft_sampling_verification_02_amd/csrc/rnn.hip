// rnn.hip -- the RNN head's per-position gate product on gfx950.
//
// Method (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
// section 3.2, the RNN Head): a recurrent state s_k (s_0 = 0) that sees the
// whole drafted prefix.  With z = [s_{k-1}, W1[x_{k-1}], h_k] (2r + d
// entries) and one bias-free linear layer Wgco [3r, 2r + d] split into gate,
// candidate and output rows,
//   g = sigmoid(Wg z),  s_k = g * s_{k-1} + (1 - g) * tanh(Wc z),
//   e_k = tanh(Wo z),   B_k = e_k W2^T,
// so the Markov head's gathered row W1[x_{k-1}] is replaced by e_k and the
// draft step's W2 product and sampling are unchanged.  The products take
// bfloat16 operands, as the weights are: s_{k-1} and h_k are rounded to
// bfloat16 (nearest, ties to even) where they enter the gate product, e_k
// where it enters the W2 product; the state itself stays float32.
//
// rnn_hproj (once a block, before position 1): h_k is known for every
// position before the block starts, so the h part of the gate product,
// Y_h = bf16(h) Wgco[:, 2r:]^T, is one [B gamma, d] x [d, 3r] product over
// all positions: 128 x 128 output tiles staged through LDS (h converted to
// bf16 on the way), four waves of 2 x 2 bf16 32x32x16 MFMA tiles, the K
// range split so that up to 256 workgroups run in one wave; each split
// writes its own partial tile, which the gate kernel sums in split order.
//
// rnn_gate: one workgroup of 8 waves per (16 requests, 16 state entries).
// Each wave takes one eighth of the s and W1 inputs (all 2r + d inputs when
// no Y_h is given) and runs three 16x16x32 bf16 MFMA chains (gate,
// candidate and output rows of the same 16 entries), with z read straight
// from its sources and Wgco rows from the caches; the eight partial tiles
// meet in LDS and 256 threads add Y_h and apply the update.
// 256 workgroups at B = 256, r = 256.
#include "device_common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace dspark {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGateThreads = 512;
constexpr int kGateSteps = 4;  // K steps of 32 whose loads go out together
constexpr int kMaxSplits = 8;  // K splits of the precomputed h part

struct GateParams {
    const float *s_in;  // [B, R] s_{k-1}; nullptr at k = 1 (s_0 = 0)
    float *s_out;       // [B, R] s_k
    const int32_t *xprev;  // x_{k-1} of request b at xprev[b * xprev_stride]
    int xprev_stride;
    const float *h;  // h_k of request b at h + b * h_stride
    size_t h_stride;
    const uint16_t *W1, *Wgco;
    uint16_t *e_out;  // e_k of request b at e_out + b * e_stride
    size_t e_stride;
    int32_t *idx_out;  // k = 1 only: idx_out[b] = b * gamma, the draft step's row of e_out
    int gamma, B, V, d;
    // precomputed h part: partial S of request b's row at yh + S * yh_split + (b * gamma + k - 1) * 3R
    const float *yh;   // nullptr: the gate product covers h itself
    size_t yh_split;
    int yS, kpos;      // splits, k - 1
};

// float32 -> bfloat16 bits, nearest with ties to even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint4 pack8(const float4 &a, const float4 &b) {
    return make_uint4(bf16_bits(a.x) | (bf16_bits(a.y) << 16), bf16_bits(a.z) | (bf16_bits(a.w) << 16),
                      bf16_bits(b.x) | (bf16_bits(b.y) << 16), bf16_bits(b.z) | (bf16_bits(b.w) << 16));
}

// entries kk .. kk + 7 of z for request b (kk a multiple of 8, so the eight
// lie in one of the three parts).  Both loads are issued whatever the part
// (the float32 one from a valid stand-in address when the part is W1's, or
// s_0 = 0), and the part is selected after: loads inside branches would make
// the compiler wait for them at every join.
template <int R>
__device__ __forceinline__ uint4 z8(const GateParams &p, int b, int prev, int kk) {
    const uint16_t *w1row = p.W1 + size_t(prev) * R;
    const bool in_s = kk < R, in_w1 = !in_s && kk < 2 * R;
    const float *stand_in = reinterpret_cast<const float *>(w1row);  // 2R >= 32 bytes
    const float *fsrc = in_s ? (p.s_in ? p.s_in + size_t(b) * R + kk : stand_in)
                             : (in_w1 ? stand_in : p.h + size_t(b) * p.h_stride + (kk - 2 * R));
    const uint4 w = *reinterpret_cast<const uint4 *>(w1row + min(max(kk - R, 0), R - 8));
    const float4 f0 = reinterpret_cast<const float4 *>(fsrc)[0], f1 = reinterpret_cast<const float4 *>(fsrc)[1];
    const uint4 z = in_w1 ? w : pack8(f0, f1);
    return (in_s && !p.s_in) ? make_uint4(0u, 0u, 0u, 0u) : z;
}

__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// MFMA 16x16x32 layout: lane l supplies row l % 16 of A (a request) and
// column l % 16 of B (a gate entry), entries 8 (l / 16) .. + 7 of the K step;
// it receives D rows 4 (l / 16) .. + 3 of column l % 16.
template <int R>
__global__ __launch_bounds__(kGateThreads) void rnn_gate_kernel(GateParams p) {
    constexpr int NCB = R / 16;  // blocks of 16 state entries
    constexpr int NW = kGateThreads / 64;
    const int ct = blockIdx.x % NCB, bt = blockIdx.x / NCB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = 2 * R + p.d;                // Wgco row length
    const int nks = (p.yh ? 2 * R : K) >> 5;  // K steps this kernel runs
    const int m = lane & 15, grp = lane >> 4;
    const int b = min(bt * 16 + m, p.B - 1);  // rows past the batch repeat its last request
    const int prev = min(max(p.xprev[size_t(b) * p.xprev_stride], 0), p.V - 1);
    const int c0 = ct * 16;
    const uint16_t *wg = p.Wgco + size_t(c0 + m) * K;
    const uint16_t *wc = wg + size_t(R) * K;
    const uint16_t *wo = wc + size_t(R) * K;
    const int s0 = (nks * wave) / NW, s1 = (nks * (wave + 1)) / NW;
    // the update's own inputs (threads 0..255, one (request, entry) each):
    // loaded before the product so that their latency overlaps it
    const int ul = tid & 63, uv = (tid >> 6) & 3;
    const int urow = bt * 16 + 4 * (ul >> 4) + uv, ucol = c0 + (ul & 15);
    const bool upd = tid < 256 && urow < p.B;
    const int ur = min(urow, p.B - 1);
    float yg = 0.f, yc = 0.f, yo = 0.f;
    if (p.yh) {
        const float *y = p.yh + (size_t(ur) * p.gamma + p.kpos) * (3 * R) + ucol;
        float t[kMaxSplits][3];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) {
            const float *ys = y + size_t(min(sp, p.yS - 1)) * p.yh_split;
            t[sp][0] = ys[0];
            t[sp][1] = ys[R];
            t[sp][2] = ys[2 * R];
        }
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) {
            yg += sp < p.yS ? t[sp][0] : 0.f;
            yc += sp < p.yS ? t[sp][1] : 0.f;
            yo += sp < p.yS ? t[sp][2] : 0.f;
        }
    }
    const float sprev = p.s_in ? p.s_in[size_t(ur) * R + ucol] : 0.f;
    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, ac = ag, ao = ag;
    for (int st = s0; st < s1; st += kGateSteps) {
        uint4 za[kGateSteps], xg[kGateSteps], xc[kGateSteps], xo[kGateSteps];
#pragma unroll
        for (int u = 0; u < kGateSteps; ++u) {
            const int su = min(st + u, s1 - 1);  // past the wave's share: reloaded, zeroed below
            const int kk = 32 * su + 8 * grp;
            za[u] = z8<R>(p, b, prev, kk);
            xg[u] = *reinterpret_cast<const uint4 *>(wg + kk);
            xc[u] = *reinterpret_cast<const uint4 *>(wc + kk);
            xo[u] = *reinterpret_cast<const uint4 *>(wo + kk);
        }
#pragma unroll
        for (int u = 0; u < kGateSteps; ++u) {
            if (st + u >= s1) za[u] = make_uint4(0u, 0u, 0u, 0u);
            ag = mfma16(za[u], xg[u], ag);
            ac = mfma16(za[u], xc[u], ac);
            ao = mfma16(za[u], xo[u], ao);
        }
    }
    __shared__ float part[NW][3][64][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        part[wave][0][lane][v] = ag[v];
        part[wave][1][lane][v] = ac[v];
        part[wave][2][lane][v] = ao[v];
    }
    __syncthreads();
    if (upd) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            yg += part[w][0][ul][uv];
            yc += part[w][1][ul][uv];
            yo += part[w][2][ul][uv];
        }
        const float g = 1.0f / (1.0f + expf(-yg));
        p.s_out[size_t(urow) * R + ucol] = g * sprev + (1.0f - g) * tanhf(yc);
        p.e_out[size_t(urow) * p.e_stride + ucol] = uint16_t(bf16_bits(tanhf(yo)));
    }
    if (p.idx_out && ct == 0 && tid < 16 && bt * 16 + tid < p.B) p.idx_out[bt * 16 + tid] = (bt * 16 + tid) * p.gamma;
}

constexpr int kProjTile = 128;  // output tile edge
constexpr int kProjBK = 64;     // K entries a stage (a multiple of 32)
constexpr int kProjPad = kProjBK + 8;  // LDS row length in bf16: rows 16 bytes apart from a bank multiple
constexpr int kProjA = kProjTile * kProjBK / 4 / 256;  // float4 loads of h a thread a stage
constexpr int kProjB = kProjTile * kProjBK / 8 / 256;  // uint4 loads of Wgco a thread a stage

struct HprojParams {
    const float *h;        // [M, d]
    const uint16_t *Wgco;  // [N, 2R + d]; the h part of row j starts at column 2R
    float *y;              // [S, M, N]
    int M, N, d, K, R, kchunk;
};

// C[m][j] = sum_i bf16(h[m][i]) Wgco[j][2R + i] over this workgroup's K
// split, for a 128 x 128 tile.  Wave w computes rows 64 (w / 2) .. + 63 and
// columns 64 (w % 2) .. + 63 as 2 x 2 MFMA tiles; each 64-wide K stage is
// staged in LDS (double-buffered) by the whole workgroup while the next one
// is loaded into registers.  K splits are multiples of 32, so a split's
// last stage may hold fewer entries (a multiple of 32): its loads past them
// repeat the last group and are not used.
__global__ __launch_bounds__(256) void rnn_hproj_kernel(HprojParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kProjTile][kProjPad];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kProjTile][kProjPad];
    const int nb = (p.N + kProjTile - 1) / kProjTile, mb = (p.M + kProjTile - 1) / kProjTile;
    const int bn = blockIdx.x % nb, bm = (blockIdx.x / nb) % mb, sk = blockIdx.x / (nb * mb);
    const int m0 = bm * kProjTile, n0 = bn * kProjTile;
    const int k_lo = sk * p.kchunk, k_hi = min(p.d, k_lo + p.kchunk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wr = 64 * (wave >> 1), wc = 64 * (wave & 1);
    // staging slots: A kProjA float4 a thread (row idx / (BK / 4), columns
    // 4 (idx % (BK / 4))), B kProjB uint4 (row idx / (BK / 8), columns
    // 8 (idx % (BK / 8))); rows past the matrix repeat its last row (their
    // outputs are not written)
    constexpr int AC = kProjBK / 4, BC = kProjBK / 8;
    float4 ra[kProjA];
    uint4 rb[kProjB];
    auto load = [&](int k0) __device__ {
        const int rem = min(kProjBK, k_hi - k0);  // entries of this stage
#pragma unroll
        for (int u = 0; u < kProjA; ++u) {
            const int idx = tid + 256 * u, row = min(m0 + idx / AC, p.M - 1);
            ra[u] = *reinterpret_cast<const float4 *>(p.h + size_t(row) * p.d + k0 + min(4 * (idx % AC), rem - 4));
        }
#pragma unroll
        for (int u = 0; u < kProjB; ++u) {
            const int idx = tid + 256 * u, row = min(n0 + idx / BC, p.N - 1);
            rb[u] = *reinterpret_cast<const uint4 *>(p.Wgco + size_t(row) * p.K + 2 * p.R + k0 +
                                                     min(8 * (idx % BC), rem - 8));
        }
    };
    auto store = [&](int buf) __device__ {
#pragma unroll
        for (int u = 0; u < kProjA; ++u) {
            const int idx = tid + 256 * u;
            const uint2 v = make_uint2(bf16_bits(ra[u].x) | (bf16_bits(ra[u].y) << 16),
                                       bf16_bits(ra[u].z) | (bf16_bits(ra[u].w) << 16));
            *reinterpret_cast<uint2 *>(&As[buf][idx / AC][4 * (idx % AC)]) = v;
        }
#pragma unroll
        for (int u = 0; u < kProjB; ++u) {
            const int idx = tid + 256 * u;
            *reinterpret_cast<uint4 *>(&Bs[buf][idx / BC][8 * (idx % BC)]) = rb[u];
        }
    };
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    int buf = 0;
    if (k_lo < k_hi) {
        load(k_lo);
        store(0);
    }
    __syncthreads();
    for (int k0 = k_lo; k0 < k_hi; k0 += kProjBK) {
        const bool more = k0 + kProjBK < k_hi;
        const int nsub = min(kProjBK, k_hi - k0) / 16;  // 16-wide MFMA steps in this stage (even)
        if (more) load(k0 + kProjBK);
#pragma unroll
        for (int ks = 0; ks < kProjBK / 16; ++ks) {
            if (ks < nsub) {
                uint4 fa[2], fb[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    fa[t] = *reinterpret_cast<const uint4 *>(&As[buf][wr + 32 * t + n][16 * ks + 8 * hh]);
                    fb[t] = *reinterpret_cast<const uint4 *>(&Bs[buf][wc + 32 * t + n][16 * ks + 8 * hh]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                                            __builtin_bit_cast(bf16x8_t, fb[j]),
                                                                            acc[i][j], 0, 0, 0);
            }
        }
        // buf ^ 1 was last read in the previous stage, before the barrier
        // that closed it: one barrier a stage suffices
        if (more) store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    // value 4q + e of lane (n, hh) is row 8q + 4hh + e of the A tile, column n of the B tile
    float *y = p.y + size_t(sk) * p.M * p.N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wc + 32 * j + n;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = m0 + wr + 32 * i + 8 * q + 4 * hh + e;
                    if (row < p.M && col < p.N) y[size_t(row) * p.N + col] = acc[i][j][4 * q + e];
                }
        }
}

}  // namespace

RnnProjPlan rnn_proj_plan(int B, int gamma, int r, int d) {
    RnnProjPlan pl{};
    const long long M = 1LL * B * gamma, N = 3LL * r;
    // worth it once the h part dominates the per-position product: measured
    // at B = 256, r = 256, gamma = 5, a block's draft takes 5.5 us less with
    // it at d = 1024, and as much or less at d = 2048 and 4096
    if (d < 4 * r || gamma < 2) return pl;
    const long long tiles = ((M + kProjTile - 1) / kProjTile) * ((N + kProjTile - 1) / kProjTile);
    const int ksteps = d / 32;
    // as many K splits as fit one workgroup a CU (256 CUs), at most
    // kMaxSplits (the gate kernel sums them)
    int S = int(std::max(1LL, std::min<long long>(std::min(ksteps, kMaxSplits), 256 / tiles)));
    const int kchunk = 32 * ((ksteps + S - 1) / S);
    S = (d + kchunk - 1) / kchunk;
    if (size_t(S) * M * N * 4 > (size_t(512) << 20)) return pl;  // too large: the gate kernel covers h itself
    pl.S = S;
    pl.kchunk = kchunk;
    pl.blocks = int(tiles * S);
    pl.floats = size_t(S) * M * N;
    return pl;
}

hipError_t launch_rnn_hproj(const float *h, const uint16_t *Wgco, float *y, int B, int gamma, int r, int d,
                            const RnnProjPlan &pl, hipStream_t s) {
    HprojParams p{h, Wgco, y, B * gamma, 3 * r, d, 2 * r + d, r, pl.kchunk};
    launch_kernel("rnn_hproj", rnn_hproj_kernel, dim3(pl.blocks), dim3(256), s, p);
    return hipGetLastError();
}

hipError_t launch_rnn_gate(const RnnGateArgs &a, hipStream_t s) {
    GateParams p{};
    p.s_in = a.s_in;
    p.s_out = a.s_out;
    p.xprev = a.xprev;
    p.xprev_stride = a.xprev_stride;
    p.h = a.h;
    p.h_stride = a.h_stride;
    p.W1 = a.W1;
    p.Wgco = a.Wgco;
    p.e_out = a.e_out;
    p.e_stride = a.e_stride;
    p.idx_out = a.idx_out;
    p.yh = a.yh;
    p.yh_split = a.yh_split;
    p.yS = a.yS;
    p.kpos = a.kpos;
    p.gamma = a.gamma;
    p.B = a.B;
    p.V = a.V;
    p.d = a.d;
    const int nbt = (a.B + 15) / 16;
    const dim3 block(kGateThreads);
    switch (a.r) {
        case 16: launch_kernel("rnn_gate", rnn_gate_kernel<16>, dim3(nbt * 1), block, s, p); break;
        case 32: launch_kernel("rnn_gate", rnn_gate_kernel<32>, dim3(nbt * 2), block, s, p); break;
        case 64: launch_kernel("rnn_gate", rnn_gate_kernel<64>, dim3(nbt * 4), block, s, p); break;
        case 128: launch_kernel("rnn_gate", rnn_gate_kernel<128>, dim3(nbt * 8), block, s, p); break;
        case 256: launch_kernel("rnn_gate", rnn_gate_kernel<256>, dim3(nbt * 16), block, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dspark
