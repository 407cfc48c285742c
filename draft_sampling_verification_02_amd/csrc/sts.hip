// sts.hip -- sequential temperature scaling of the confidence head on gfx950.
//
// Method (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
// section 4.2): the confidences are calibrated left to right, position by
// position, each with a one-dimensional grid search for the temperature that
// minimises the expected calibration error (ECE) of the prefix survival
// product, the earlier positions' temperatures held fixed.  Here:
//   c'_k = sigmoid(logit(c_k) / tau_k)  (order-preserving for tau > 0),
//   a'_k = c'_1 ... c'_k,   outcome y_k = [n >= k]  (drafts 1..k accepted),
//   ECE_k(tau) = sum over M equal-width bins of |sum y - sum a'| / N_k,
// over the N_k samples that verified position k (ell >= k); the first grid
// value with the smallest ECE wins; a position nobody verified keeps tau = 1.
//
// Kernels, per position k (after one that clears the accumulators):
//   sts_hist  one workgroup per 256 samples, one sample a thread: it first
//             advances its sample's a' by position k - 1's chosen tau, then
//             for every grid value bins a'_{k-1} c'_k and adds it to an LDS
//             histogram per (grid value, bin) -- a' in 2^-32 fixed point and
//             the outcomes as counts, so the integer sums are the same in any
//             order -- and finally adds the histogram into global per-position
//             accumulators.
//   sts_pick  one workgroup: every grid value's ECE in double precision from
//             the accumulators, the first minimum, tau_k and its ECE.
#include "device_common.hpp"
#include "internal.hpp"

namespace dspark {

namespace {

constexpr int kStsThreads = 256;
constexpr int kPickThreads = 1024;

struct StsParams {
    const float *c;  // [N, gamma]
    const int32_t *n, *ell;
    const float *grid;
    int N, gamma, G, M, k;
    float *a;               // [N] a'_{k-1}, advanced in place
    const float *tau;       // [gamma] chosen temperatures (k - 1 read)
    unsigned long long *acc_p;  // [gamma, G, M] sum of a' * 2^32
    uint32_t *acc_y;        // [gamma, G, M] outcome counts
    uint32_t *acc_n;        // [gamma] samples that verified the position
    float *tau_out, *ece_out, *ece_grid;
};

__device__ __forceinline__ float logit_of(float c) { return logf(c) - log1pf(-c); }

__global__ __launch_bounds__(256) void sts_clear_kernel(StsParams p) {
    const size_t n = size_t(p.gamma) * p.G * p.M;
    for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256) {
        p.acc_p[i] = 0ull;
        p.acc_y[i] = 0u;
    }
    if (blockIdx.x == 0 && int(threadIdx.x) < p.gamma) p.acc_n[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(kStsThreads) void sts_hist_kernel(StsParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    unsigned long long *hp = reinterpret_cast<unsigned long long *>(lds);  // [G, M]
    uint32_t *hy = reinterpret_cast<uint32_t *>(hp + size_t(p.G) * p.M);   // [G, M]
    float *gv = reinterpret_cast<float *>(hy + size_t(p.G) * p.M);          // [G]
    __shared__ uint32_t valid_count;
    const int tid = threadIdx.x;
    const int GM = p.G * p.M;
    for (int i = tid; i < GM; i += kStsThreads) {
        hp[i] = 0ull;
        hy[i] = 0u;
    }
    for (int g = tid; g < p.G; g += kStsThreads) gv[g] = p.grid[g];
    if (tid == 0) valid_count = 0u;
    const int i = blockIdx.x * kStsThreads + tid;
    const bool in = i < p.N;
    const int ic = in ? i : 0;
    const int L = p.ell ? p.ell[ic] : p.gamma;
    const bool valid = in && L >= p.k && L <= p.gamma;
    float a = 1.0f;
    if (p.k > 1) {
        // advance a' by position k - 1 (its temperature was chosen by the last
        // pick); a'_0 = 1, so the buffer is first read at k = 3
        a = p.k > 2 ? p.a[ic] : 1.0f;
        const float lg = logit_of(p.c[size_t(ic) * p.gamma + p.k - 2]);
        a = a / (1.0f + expf(-lg / p.tau[p.k - 2]));
        if (in) p.a[i] = a;
    }
    const float lg = logit_of(p.c[size_t(ic) * p.gamma + p.k - 1]);
    const uint32_t y = p.n[ic] >= p.k ? 1u : 0u;
    __syncthreads();
    if (valid) {
        atomicAdd(&valid_count, 1u);
        for (int g = 0; g < p.G; ++g) {
            const float t = gv[g];
            if (!(t > 0.f)) continue;
            const float pr = a / (1.0f + expf(-lg / t));
            const int m = min(max(int(pr * float(p.M)), 0), p.M - 1);  // NaN converts to 0
            atomicAdd(&hp[g * p.M + m], __float2ull_rn(pr * 4294967296.0f));
            if (y) atomicAdd(&hy[g * p.M + m], 1u);
        }
    }
    __syncthreads();
    const size_t base = size_t(p.k - 1) * GM;
    for (int j = tid; j < GM; j += kStsThreads) {
        if (hp[j]) atomicAdd(&p.acc_p[base + j], hp[j]);
        if (hy[j]) atomicAdd(&p.acc_y[base + j], hy[j]);
    }
    if (tid == 0 && valid_count) atomicAdd(&p.acc_n[p.k - 1], valid_count);
}

__global__ __launch_bounds__(kPickThreads) void sts_pick_kernel(StsParams p) {
    __shared__ double be[kPickThreads];
    __shared__ int bi[kPickThreads];
    const int tid = threadIdx.x;
    const uint32_t Nk = p.acc_n[p.k - 1];
    const size_t base = size_t(p.k - 1) * p.G * p.M;
    double best = __builtin_inf();
    int bg = 0x7fffffff;
    for (int g = tid; g < p.G; g += kPickThreads) {
        double e = __builtin_inf();
        if (p.grid[g] > 0.f && Nk > 0) {
            e = 0.0;
            for (int m = 0; m < p.M; ++m) {
                const double sp = double(p.acc_p[base + size_t(g) * p.M + m]) * (1.0 / 4294967296.0);
                const double sy = double(p.acc_y[base + size_t(g) * p.M + m]);
                e += fabs(sy - sp);
            }
            e /= double(Nk);
        }
        if (p.ece_grid) p.ece_grid[size_t(p.k - 1) * p.G + g] = float(e);
        if (e < best) {  // g rises within a thread: the first minimum stays
            best = e;
            bg = g;
        }
    }
    be[tid] = best;
    bi[tid] = bg;
    __syncthreads();
    for (int o = kPickThreads / 2; o > 0; o >>= 1) {
        if (tid < o) {
            const double e2 = be[tid + o];
            const int g2 = bi[tid + o];
            if (e2 < be[tid] || (e2 == be[tid] && g2 < bi[tid])) {
                be[tid] = e2;
                bi[tid] = g2;
            }
        }
        __syncthreads();
    }
    if (tid == 0) {
        const bool none = Nk == 0 || bi[0] == 0x7fffffff;
        p.tau_out[p.k - 1] = none ? 1.0f : p.grid[bi[0]];
        p.ece_out[p.k - 1] = none ? __builtin_nanf("") : float(be[0]);
    }
}

}  // namespace

StsPlan sts_plan(int N, int gamma, int G, int M) {
    StsPlan p{};
    p.blocks = (N + kStsThreads - 1) / kStsThreads;
    p.lds = size_t(G) * M * (8 + 4) + size_t(G) * 4;
    (void)gamma;
    return p;
}

StsWork sts_carve(void *ws, int N, int gamma, int G, int M, size_t *bytes) {
    Carve c(ws);
    StsWork w{};
    w.a = c.take<float>(N);
    w.acc_p = c.take<unsigned long long>(size_t(gamma) * G * M);
    w.acc_y = c.take<uint32_t>(size_t(gamma) * G * M);
    w.acc_n = c.take<uint32_t>(gamma);
    if (bytes) *bytes = c.off + 256;
    return w;
}

hipError_t launch_sts(const StsArgs &a, const StsPlan &pl, const StsWork &w, hipStream_t s) {
    StsParams p{};
    p.c = a.c;
    p.n = a.n;
    p.ell = a.ell;
    p.grid = a.grid;
    p.N = a.N;
    p.gamma = a.gamma;
    p.G = a.G;
    p.M = a.M;
    p.a = w.a;
    p.tau = a.tau_out;
    p.acc_p = w.acc_p;
    p.acc_y = w.acc_y;
    p.acc_n = w.acc_n;
    p.tau_out = a.tau_out;
    p.ece_out = a.ece_out;
    p.ece_grid = a.ece_grid;
    launch_kernel("sts_clear", sts_clear_kernel, dim3(64), dim3(256), s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int k = 1; k <= a.gamma; ++k) {
        p.k = k;
        const ProfEvents ev = prof_events("sts_hist");
        hipExtLaunchKernelGGL(sts_hist_kernel, dim3(pl.blocks), dim3(kStsThreads), uint32_t(pl.lds), s, ev.start,
                              ev.stop, 0, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        launch_kernel("sts_pick", sts_pick_kernel, dim3(1), dim3(kPickThreads), s, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dspark
