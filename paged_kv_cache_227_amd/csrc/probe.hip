// probe.hip -- measurement kernels beside the decode path.
//
// probe_read: every thread streams 16-byte vectors (grid-stride, 4 loads in
// flight per iteration) and folds them into an xor checksum, one word per
// workgroup; gives the HBM read rate a plain coalesced kernel reaches.
// probe_copy: a plain 16-byte copy, a kernel of known traffic (bytes read =
// bytes written = size) for calibrating hardware counters.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 4096;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* src, size_t n, float* sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const uint4 a = src[i];
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ uint32_t red[kProbeThreads / kWave];
    for (int m = 1; m < kWave; m <<= 1) x ^= __shfl_xor(x, m, kWave);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int k = 0; k < kProbeThreads / kWave; ++k) t ^= red[k];
        sink[blockIdx.x] = __uint_as_float(t);
    }
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4* src, uint4* dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
    return hipGetLastError();
}

}  // namespace pkv
