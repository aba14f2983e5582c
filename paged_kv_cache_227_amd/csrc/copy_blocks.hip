// copy_blocks.hip -- the data half of copy-on-write.
//
// A sequence about to write into a block that other sequences also hold first
// receives a private block from the host's block manager ("How a serving
// engine actually works", paperfordummies.in, section "Copy-on-write, because
// you have used fork()"); the tokens the shared block already holds for it,
// its first n rows, must be in the private block before the write lands.
// Rows 0 .. n-1 of a [B][n_kv_heads][head_dim] block are one contiguous run of
// n * row_bytes bytes, so each copy is a contiguous move inside the cache.
//
// Grid: (n_copies * chunks, 2) -- y selects the K or the V cache.  A workgroup
// of 256 threads moves one chunk (256 x U vectors) of one copy, with
// nontemporal stores (the target is read next by a streaming decode, not from
// cache).  Two shapes, chosen by the most a call can move:
//   - more than the 256 MB last-level cache: one 16-byte vector per thread and
//     nontemporal loads -- the sources cannot be cache resident, so the copy
//     streams (many small workgroups keep the most requests in flight);
//   - otherwise two vectors per thread and ordinary loads, which hit when the
//     source blocks were touched recently (a fork copies the block the prompt
//     just wrote).
// The vectors are the compiler's native 4 x 32-bit type: with HIP's uint4
// struct in the guarded loads the compiler waits for each load before issuing
// the next.  A copy whose blocks or row count lie outside their ranges is
// skipped: the kernel never touches memory outside the two caches and the
// three index arrays.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int64_t kCopyStreamBytes = (int64_t)256 << 20;

template <int VB>
struct CopyVec;
template <>
struct CopyVec<16> {
    using T = v4u32_t;
};
template <>
struct CopyVec<4> {
    using T = uint32_t;
};
template <>
struct CopyVec<2> {
    using T = uint16_t;
};

template <int VB, int U>
constexpr int64_t copy_chunk_bytes() {
    return (int64_t)kCopyThreads * U * VB;
}

template <int VB, int U, bool STREAM>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyParams p) {
    using T = typename CopyVec<VB>::T;
    constexpr int64_t CHUNK = copy_chunk_bytes<VB, U>();
    const int i = blockIdx.x / p.chunks;
    const int c = blockIdx.x - i * p.chunks;
    const int src = p.src_blocks[i];
    const int dst = p.dst_blocks[i];
    const int n = p.n_rows[i];
    if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks || n <= 0 || n > p.block_size) return;
    const int64_t bytes = (int64_t)n * p.row_bytes;
    const int64_t lo = (int64_t)c * CHUNK;
    if (lo >= bytes) return;
    const int64_t hi = lo + CHUNK < bytes ? lo + CHUNK : bytes;
    const int64_t blk_bytes = (int64_t)p.block_size * p.row_bytes;
    char* cache = static_cast<char*>(blockIdx.y ? p.v_cache : p.k_cache);
    const char* from = cache + (int64_t)src * blk_bytes;
    char* to = cache + (int64_t)dst * blk_bytes;
    T r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t off = lo + (int64_t)(threadIdx.x + u * kCopyThreads) * VB;
        if (off < hi) {
            if constexpr (STREAM)
                r[u] = __builtin_nontemporal_load(reinterpret_cast<const T*>(from + off));
            else
                r[u] = *reinterpret_cast<const T*>(from + off);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t off = lo + (int64_t)(threadIdx.x + u * kCopyThreads) * VB;
        if (off < hi) __builtin_nontemporal_store(r[u], reinterpret_cast<T*>(to + off));
    }
}

template <int VB, int U, bool STREAM>
static hipError_t launch_copy_shape(CopyParams p, hipStream_t stream) {
    const int64_t blk_bytes = (int64_t)p.block_size * p.row_bytes;
    const int64_t chunks = (blk_bytes + copy_chunk_bytes<VB, U>() - 1) / copy_chunk_bytes<VB, U>();
    if (chunks * p.n_copies > 0x7fffffff) return hipErrorInvalidConfiguration;
    p.chunks = (int32_t)chunks;
    hipLaunchKernelGGL((copy_blocks_kernel<VB, U, STREAM>), dim3((unsigned)(chunks * p.n_copies), 2),
                       dim3(kCopyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream) {
    if (p.n_copies <= 0) return hipSuccess;
    // the most this call can read: every copy a whole block, both caches
    const bool stream_it = (int64_t)p.n_copies * p.block_size * p.row_bytes * 2 > kCopyStreamBytes;
    if (p.row_bytes % 16 == 0)
        return stream_it ? launch_copy_shape<16, 1, true>(p, stream) : launch_copy_shape<16, 2, false>(p, stream);
    if (p.row_bytes % 4 == 0) return launch_copy_shape<4, 4, false>(p, stream);
    return launch_copy_shape<2, 8, false>(p, stream);
}

}  // namespace pkv
