// pkv_launch.h -- parameter blocks and launchers shared between the C-ABI
// wrapper (pagedkv_abi.hip) and the kernel sources.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct AppendParams {
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int32_t* block_tables;
    const int32_t* positions;
    int32_t num_blocks;
    int32_t block_size;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t row_bytes;  // n_kv_heads * head_dim * element bytes
};

struct AppendTokensParams {
    const void* k_new;  // [total][n_kv_heads][head_dim]
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int32_t* block_tables;
    const int32_t* cu_new;     // [num_seqs + 1]: sequence s owns rows cu_new[s] .. cu_new[s+1]-1
    const int32_t* start_pos;  // [num_seqs]: position of each sequence's first new row
    int32_t num_blocks;
    int32_t block_size;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t total;      // rows in k_new (the host's cu_new[num_seqs])
    int32_t row_bytes;  // n_kv_heads * head_dim * element bytes
};

struct PrefillParams {
    const void* q;  // [total][n_q_heads][head_dim]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* cu_q;          // [num_seqs + 1]
    const int32_t* context_lens;  // [num_seqs]: tokens in the cache, the chunk included
    void* out;                    // [total][n_q_heads][head_dim]
    int32_t num_blocks;
    int32_t n_kv_heads;
    int32_t n_q_heads;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t max_q_len;    // longest chunk (sizes the grid)
    int32_t block_shift;  // log2 of the block size (8 .. 64 tokens)
    float scale_log2;     // scale * log2(e)
};

struct SwapParams {
    void* k_cache;
    void* v_cache;
    const int32_t* blocks;  // [n]: the block of each host slot
    void* host_k;           // device view of pinned host buffers [n][block bytes]
    void* host_v;
    int32_t num_blocks;
    int32_t n;
    int32_t chunks;     // workgroups per block (set by the launcher)
    int64_t blk_bytes;  // block_size * n_kv_heads * head_dim * element bytes (a multiple of 16)
};

struct CopyParams {
    void* k_cache;
    void* v_cache;
    const int32_t* src_blocks;
    const int32_t* dst_blocks;
    const int32_t* n_rows;
    int32_t num_blocks;
    int32_t block_size;
    int32_t n_copies;
    int32_t chunks;     // workgroups per copy (set by the launcher)
    int64_t row_bytes;  // n_kv_heads * head_dim * element bytes
};

// The flat schedule's grid never has more waves than this; its workspace is
// sized for it.
constexpr int kMaxFlatWorkers = 8192;
// Most teams in a period of the flat schedule (two workgroups of at most 8
// waves); the schedule header holds their offsets.
constexpr int kMaxFlatPeriod = 16;
// Largest batch the flat schedule serves (its per-workgroup LDS holds two
// int32 per sequence); larger batches use fixed partitions.
constexpr int kMaxFlatSeqs = 8000;
// Most adjacent KV heads one wave streams together; the workspace is sized for it.
constexpr int kMaxHeadsPerWave = 2;

struct DecodeParams {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    void* out;
    // Split-K workspace.  Fixed partitions: ws_acc [num_seqs][n_q_heads][n_parts_max][head_dim],
    // ws_ml [..][2] (running max in log2 units, sum).  Flat schedule: records
    // [num_seqs * n_kv_heads + kMaxFlatWorkers][G][head_dim] and [..][G][2], and
    // ws_hdr = {tiles per period, teams per period Q, tile prefix per sequence
    // [num_seqs + 1], the teams' offsets in a period [Q + 1]}.
    float* ws_acc;
    float* ws_ml;
    int32_t* ws_hdr;
    int32_t num_blocks;
    int32_t n_kv_heads;
    int32_t n_q_heads;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t part_tokens;  // 0 selects the flat schedule
    int32_t n_parts_max;
    int32_t min_tiles_per_worker;
    int32_t heads_per_wave;  // adjacent KV heads one wave streams together (see decode_heads_per_wave)
    int32_t team;            // waves walking the same blocks, one head group each (set by the launchers)
    int32_t split_pct;       // flat schedule: the first team of a workgroup's share of its tiles (set by the launcher)
    int32_t xcd_pct;         // flat schedule: an even workgroup's share of it and the next one's tiles (set by the launcher)
    int32_t block_shift;     // log2 of the cache block size (8, 16, 32 or 64 tokens)
    float scale_log2;  // scale * log2(e): scores are kept in base-2 units
    // A fused append (flat schedule only; positions == nullptr otherwise): the
    // decode pass reads each sequence's new row from k_new / v_new ([num_seqs]
    // [n_kv_heads][head_dim]) at positions[s], and the merge pass writes it to
    // its slot in k_cache_w / v_cache_w (the same caches).
    const void* k_new;
    const void* v_new;
    const int32_t* positions;
    void* k_cache_w;
    void* v_cache_w;
};

// Each returns hipSuccess or the launch error.  dtype: 0 f32, 1 f16, 2 bf16.
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream);
hipError_t launch_swap(SwapParams p, bool to_cache, hipStream_t stream);
hipError_t launch_append_tokens(const AppendTokensParams& p, hipStream_t stream);
// Prefill grid: (KV head, tile of kPrefillRows query rows, sequence); a grid's
// second and third dimensions hold at most 65535.
constexpr int kPrefillRows = 128;
constexpr int64_t kMaxPrefillTiles = 65535;
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int group, hipStream_t stream);
bool prefill_supported(int dtype, int head_dim, int group);
hipError_t launch_decode_partitions(const DecodeParams& p, int dtype, int head_dim, int group,
                                    hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams& p, int dtype, int head_dim, int group, hipStream_t stream);
bool decode_supported(int dtype, int head_dim, int group);
// KV heads per wave the decode kernels use for this shape (1 or 2).
int decode_heads_per_wave(int dtype, int head_dim, int group, int n_kv_heads);

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace pkv
