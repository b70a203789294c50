// HBM stream-read ceiling: a whole-GPU grid reads a buffer once, 16 bytes per
// lane per load in a grid-stride loop, and folds what it read into
// one XOR word per workgroup (so the loads cannot be dropped, and the result is
// checkable). Used to measure the read bandwidth the kernels here are compared
// against, next to the vendor peak.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4 *__restrict__ buf, int64_t n16,
                                                                     uint32_t *__restrict__ xor_out) {
    __shared__ uint32_t s_x[kStreamThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i < n16; i += stride) {
        const uint4 a = buf[i];
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
    if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kStreamThreads / 64; ++w) r ^= s_x[w];
        xor_out[blockIdx.x] = r;
    }
}

int launch_stream_read(const void *buf, size_t bytes, uint32_t *xor_out, hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadBlocks), dim3(kStreamThreads), 0, stream,
                       (const uint4 *)buf, (int64_t)(bytes / 16), xor_out);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace sa
