// swap.hip -- swap a preempted sequence's cache blocks out to pinned host
// memory and back.
//
// When no block is free and no sequence can grow, a victim is preempted whole
// ("How a serving engine actually works", paperfordummies.in, section "When
// there are no free blocks left"); it comes back either by recomputing its
// cache or by swapping: copying its blocks to host memory and later back,
// which costs bandwidth twice ("Paged Attention and the Block Manager",
// snowch.github.io ch08, "Running out of memory becomes a scheduling
// decision").  Slot i of the host buffers holds block blocks[i] of each cache
// ([n][B][n_kv_heads][head_dim], whole blocks); swap-in writes slot i into
// block blocks[i], which need not be the block it came from.
//
// The GPU moves the data itself, through the device mapping of the pinned host
// buffers: scattered blocks need no staging copy and no per-block DMA call.
// Grid (n * chunks, 2) -- y selects the K or the V cache; a workgroup moves one
// chunk (256 x 4 vectors of 16 bytes) of one block, its four loads in flight
// before its stores.  A block index outside the pool skips that slot.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 4;
constexpr int64_t kSwapChunk = (int64_t)kSwapThreads * kSwapUnroll * 16;

template <bool TO_CACHE>
__global__ __launch_bounds__(kSwapThreads) void swap_kernel(SwapParams p) {
    const int i = blockIdx.x / p.chunks;
    const int c = blockIdx.x - i * p.chunks;
    const int b = p.blocks[i];
    if (b < 0 || b >= p.num_blocks) return;
    const int64_t lo = (int64_t)c * kSwapChunk;
    const int64_t hi = lo + kSwapChunk < p.blk_bytes ? lo + kSwapChunk : p.blk_bytes;
    char* cache = static_cast<char*>(blockIdx.y ? p.v_cache : p.k_cache) + (int64_t)b * p.blk_bytes;
    char* host = static_cast<char*>(blockIdx.y ? p.host_v : p.host_k) + (int64_t)i * p.blk_bytes;
    const char* from = TO_CACHE ? host : cache;
    char* to = TO_CACHE ? cache : host;
    v4u32_t r[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
        const int64_t off = lo + (int64_t)(threadIdx.x + u * kSwapThreads) * 16;
        if (off < hi) r[u] = *reinterpret_cast<const v4u32_t*>(from + off);
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
        const int64_t off = lo + (int64_t)(threadIdx.x + u * kSwapThreads) * 16;
        if (off < hi) *reinterpret_cast<v4u32_t*>(to + off) = r[u];
    }
}

hipError_t launch_swap(SwapParams p, bool to_cache, hipStream_t stream) {
    if (p.n <= 0) return hipSuccess;
    const int64_t chunks = (p.blk_bytes + kSwapChunk - 1) / kSwapChunk;
    if (chunks * p.n > 0x7fffffff) return hipErrorInvalidConfiguration;
    p.chunks = (int32_t)chunks;
    const dim3 grid((unsigned)(chunks * p.n), 2);
    if (to_cache)
        hipLaunchKernelGGL(swap_kernel<true>, grid, dim3(kSwapThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(swap_kernel<false>, grid, dim3(kSwapThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
