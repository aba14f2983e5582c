// append.hip -- scatter each sequence's new K/V row into its paged slot.
//
// For sequence s the new token at logical position p lands in
//     slot = block_table[s][p / B] * B + (p mod B)
// ("How a serving engine actually works", paperfordummies.in, "The one
// formula"), i.e. row (p mod B) of physical block block_table[s][p / B] of a
// [num_blocks][B][n_kv_heads][head_dim] cache.  One token's row over all KV
// heads is contiguous (n_kv_heads * head_dim elements), so the append is a
// plain bit copy of one contiguous row per sequence and per cache.
//
// Grid: (num_seqs, 2) -- y selects the K or the V cache; 256 threads copy the
// row with the widest vector the row size allows (16 bytes when it divides).
// A position or table entry outside its range skips the sequence: the kernel
// never writes outside the cache.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

template <int VB>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int s = blockIdx.x;
    const int pos = p.positions[s];
    if (pos < 0 || pos / p.block_size >= p.max_blocks) return;
    const int blk = p.block_tables[(int64_t)s * p.max_blocks + pos / p.block_size];
    if (blk < 0 || blk >= p.num_blocks) return;
    const int64_t slot = (int64_t)blk * p.block_size + pos % p.block_size;
    const bool is_v = blockIdx.y != 0;
    const char* src = static_cast<const char*>(is_v ? p.v_new : p.k_new) + (int64_t)s * p.row_bytes;
    char* dst = static_cast<char*>(is_v ? p.v_cache : p.k_cache) + slot * p.row_bytes;
    for (int off = threadIdx.x * VB; off < p.row_bytes; off += blockDim.x * VB) {
        if constexpr (VB == 16) {
            store16(dst + off, load16(src + off));
        } else if constexpr (VB == 8) {
            *reinterpret_cast<uint2*>(dst + off) = *reinterpret_cast<const uint2*>(src + off);
        } else if constexpr (VB == 4) {
            *reinterpret_cast<uint32_t*>(dst + off) = *reinterpret_cast<const uint32_t*>(src + off);
        } else {
            *reinterpret_cast<uint16_t*>(dst + off) = *reinterpret_cast<const uint16_t*>(src + off);
        }
    }
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    const dim3 grid(p.num_seqs, 2);
    const dim3 block(256);
    if (p.row_bytes % 16 == 0)
        hipLaunchKernelGGL(append_kernel<16>, grid, block, 0, stream, p);
    else if (p.row_bytes % 8 == 0)
        hipLaunchKernelGGL(append_kernel<8>, grid, block, 0, stream, p);
    else if (p.row_bytes % 4 == 0)
        hipLaunchKernelGGL(append_kernel<4>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(append_kernel<2>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
