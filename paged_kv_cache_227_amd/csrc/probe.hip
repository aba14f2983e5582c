// probe.hip -- measurement kernels beside the decode path.
//
// probe_read: each workgroup streams its own contiguous share of the buffer,
// every thread keeping 16 nontemporal 16-byte loads in flight, and folds them
// into an xor checksum, one word per workgroup: the HBM read rate a plain
// streaming kernel reaches (measured on MI355X: contiguous shares with
// nontemporal loads beat a grid-stride loop by about a quarter).
// probe_copy: a plain 16-byte copy, a kernel of known traffic (bytes read =
// bytes written = size) for calibrating hardware counters.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 4096;

constexpr int kProbeInFlight = 16;  // loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const v4u32_t* src, size_t n, float* sink) {
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n ? lo + per : n;
    uint32_t x = 0;
    size_t i = lo + threadIdx.x;
    for (; i + (kProbeInFlight - 1) * blockDim.x < hi; i += kProbeInFlight * blockDim.x) {
        v4u32_t a[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) a[u] = __builtin_nontemporal_load(src + i + u * blockDim.x);
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
    }
    for (; i < hi; i += blockDim.x) {
        const v4u32_t a = __builtin_nontemporal_load(src + i);
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
                       static_cast<const v4u32_t*>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
    return hipGetLastError();
}

}  // namespace pkv
