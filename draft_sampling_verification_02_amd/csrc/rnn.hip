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
// rnn_gate: one workgroup of 8 waves per (16 requests, 16 state entries).
// Each wave takes one eighth of the 2r + d inputs and runs three 16x16x32
// bf16 MFMA chains (gate, candidate and output rows of the same 16 entries),
// with z read straight from its three sources and Wgco rows from the caches;
// the eight partial tiles meet in LDS and 256 threads apply the update.
// 256 workgroups at B = 256, r = 256.
#include "device_common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace dspark {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGateThreads = 512;
constexpr int kGateSteps = 4;  // K steps of 32 whose loads go out together

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
    const int K = 2 * R + p.d, nks = K >> 5;
    const int m = lane & 15, grp = lane >> 4;
    const int b = min(bt * 16 + m, p.B - 1);  // rows past the batch repeat its last request
    const int prev = min(max(p.xprev[size_t(b) * p.xprev_stride], 0), p.V - 1);
    const int c0 = ct * 16;
    const uint16_t *wg = p.Wgco + size_t(c0 + m) * K;
    const uint16_t *wc = wg + size_t(R) * K;
    const uint16_t *wo = wc + size_t(R) * K;
    const int s0 = (nks * wave) / NW, s1 = (nks * (wave + 1)) / NW;
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
    if (tid < 256) {
        const int l = tid & 63, v = tid >> 6;
        float yg = 0.f, yc = 0.f, yo = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            yg += part[w][0][l][v];
            yc += part[w][1][l][v];
            yo += part[w][2][l][v];
        }
        const int row = bt * 16 + 4 * (l >> 4) + v;
        const int col = c0 + (l & 15);
        if (row < p.B) {
            const float sp = p.s_in ? p.s_in[size_t(row) * R + col] : 0.f;
            const float g = 1.0f / (1.0f + expf(-yg));
            p.s_out[size_t(row) * R + col] = g * sp + (1.0f - g) * tanhf(yc);
            p.e_out[size_t(row) * p.e_stride + col] = uint16_t(bf16_bits(tanhf(yo)));
        }
    }
    if (p.idx_out && ct == 0 && tid < 16 && bt * 16 + tid < p.B) p.idx_out[bt * 16 + tid] = (bt * 16 + tid) * p.gamma;
}

}  // namespace

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
