// debug.hip -- diagnostic kernels exposing the device random streams and the
// Gumbel transform, so tests can compare them with an independent reference.
#include "device_common.hpp"
#include "internal.hpp"

namespace dspark {

namespace {

__global__ void debug_words_kernel(uint32_t k0, uint32_t k1, uint32_t round32, int stream_id, int k, int req,
                                   int v0, int n, uint32_t *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (stream_id != kStreamAccept) {
        out[i] = noise_word(stream_id, k, uint32_t(v0 + i), uint32_t(req), round32, k0, k1);
    } else {
        out[i] = scalar_word(stream_id, k, uint32_t(req), round32, k0, k1);
    }
}

__global__ void debug_gumbel_kernel(const uint32_t *words, int n, float *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = gumbel2(words[i]);
}

}  // namespace

hipError_t launch_debug_words(uint32_t key0, uint32_t key1, uint32_t round32, int stream_id, int k, int req,
                              int v0, int n, uint32_t *out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(debug_words_kernel, dim3((n + 255) / 256), dim3(256), 0, s, key0, key1, round32, stream_id,
                       k, req, v0, n, out);
    return hipGetLastError();
}

hipError_t launch_debug_gumbel(const uint32_t *words, int n, float *out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(debug_gumbel_kernel, dim3((n + 255) / 256), dim3(256), 0, s, words, n, out);
    return hipGetLastError();
}

}  // namespace dspark
