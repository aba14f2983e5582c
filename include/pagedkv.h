/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV cache decode path.
 *
 * The operations are the two a paged KV cache needs on every decode step:
 *
 *   append  -- write each sequence's new key/value row into the slot its
 *              block table gives for the token's logical position;
 *   decode  -- attention of each sequence's query over its cached keys and
 *              values, read in place through the block table;
 *
 * and, next to them, the block copy that copy-on-write needs before an append
 * into a block that another sequence also holds, the chunked-prefill pair
 * (an n-token append and the attention of a chunk of queries), and the swap
 * of a preempted sequence's blocks to host memory and back.
 *
 * Append and decode use the address translation of "How a serving engine actually works"
 * (paperfordummies.in), section "The one formula":
 *
 *     slot(seq, i) = block_table[seq][i / B] * B + (i mod B)
 *
 * and the per-layer cache layout of "Paged-KV + Continuous Batching From
 * Scratch" (henryhe.ai), section 1, and "Paged Attention and the Block
 * Manager" (snowch.github.io ch08), section "The build": one tensor per layer,
 * indexed by physical block,
 *
 *     k_cache, v_cache : [num_blocks][block_size][n_kv_heads][head_dim]
 *
 * contiguous, element type `dtype`.  Attention itself is unchanged by paging
 * (henryhe.ai, "What's deliberately still missing": the same maths as a
 * FlashAttention forward with different addressing): for query head h of
 * sequence s, with L = context_lens[s] and KV head g = h / (n_q_heads /
 * n_kv_heads),
 *
 *     out[s][h] = sum_i softmax_i(scale * <q[s][h], K_i>) * V_i,   i < L,
 *
 * with no causal mask (a decode query attends to every cached token,
 * including its own), accumulated in fp32 and rounded to `dtype` with
 * round-to-nearest-even.  L = 0 gives a zero row.
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers unless a parameter says "host".  The caller
 *     owns every buffer it passes in; the library never allocates or frees KV
 *     blocks (that is the host block manager's job).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and return once the work is enqueued.  PKV_OK means "validated
 *     and enqueued"; faults in enqueued work surface at the caller's next
 *     synchronisation as HIP errors.
 *   - Invalid arguments return a status and leave every buffer untouched; the
 *     message of the last non-OK call on this thread is pkv_last_error().
 *     Nothing throws across this boundary.
 *   - block_tables is [num_seqs][max_blocks_per_seq] int32, row-major; entries
 *     past a sequence's last block are ignored.  Table entries outside
 *     [0, num_blocks) are a precondition violation: the kernels skip such a
 *     block (no out-of-bounds access) and the result is unspecified;
 *     pkv_validate() reports them.
 *   - Supported by the GPU path: dtype f32 / f16 / bf16, head_dim 64 or 128,
 *     n_q_heads / n_kv_heads in {1, 2, 4, 8}; block_size 8, 16, 32 or 64 for
 *     decode and prefill (the block size is "the one tuning knob" of "How a
 *     serving engine actually works", section "The one formula"), any for the
 *     appends, block copies and swaps.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_EINVAL = 1,  /* bad pointer, size, shape or layout */
    PKV_ENOTSUP = 2, /* valid, but a dtype / head_dim / group size this build does not serve */
    PKV_EHIP = 3,    /* the HIP runtime returned an error */
    PKV_EOOB = 4     /* pkv_validate: a table entry or position out of range */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* Shape of one layer's cache pair (host struct, read during the call only). */
typedef struct {
    int32_t num_blocks; /* physical blocks in the pool */
    int32_t block_size; /* tokens per block (B): 8, 16, 32 or 64 for attention, any for copies */
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t dtype; /* pkv_dtype */
} pkv_layout;

/*
 * paged_kv_append -- scatter each sequence's new token into its slot.
 *
 * For every s < num_seqs, with p = positions[s]:
 *     k_cache[slot(s, p)][:][:] = k_new[s][:][:]   (and likewise for v)
 * a bit-exact copy.  Nothing else in the caches changes.
 *
 *   k_new, v_new  [num_seqs][n_kv_heads][head_dim], element type layout->dtype
 *   k_cache, v_cache  the layer's caches (see top of file), written in place
 *   layout        host pointer
 *   block_tables  [num_seqs][max_blocks_per_seq] int32
 *   positions     [num_seqs] int32: logical index of each new token; the host
 *                 must have grown the table to cover it (p / B < blocks held)
 *
 * Preconditions: the target slots are pairwise distinct (a writer owns its
 * block: copy-on-write happens on the host before the append).  A position
 * outside [0, max_blocks_per_seq * B) or a table entry outside the pool makes
 * the kernel skip that sequence.
 */
pkv_status paged_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const pkv_layout* layout, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* positions, int32_t num_seqs,
                           void* stream);

/*
 * paged_kv_swap_out / paged_kv_swap_in -- swap a preempted sequence's cache.
 *
 * When no block is free and no sequence can grow, a victim is preempted whole
 * and comes back later either by recomputing its cache (prefill) or by having
 * its blocks swapped to host memory and back ("How a serving engine actually
 * works", paperfordummies.in, section "When there are no free blocks left";
 * "Paged Attention and the Block Manager", snowch.github.io ch08, "Running out
 * of memory becomes a scheduling decision": swapping costs bandwidth, twice).
 *
 *   swap_out:  host_k[i] = k_cache[blocks[i]], host_v[i] = v_cache[blocks[i]]
 *   swap_in:   k_cache[blocks[i]] = host_k[i], v_cache[blocks[i]] = host_v[i]
 *
 * whole blocks, bit-exact; swap-in may target other blocks than the ones
 * swapped out (the host allocator hands out whatever is free).
 *
 *   blocks          [n] int32 device array of physical blocks
 *   host_k, host_v  PINNED host buffers (hipHostMalloc, or a pinned torch
 *                   tensor) of n blocks each: [n][block_size][n_kv_heads][head_dim];
 *                   owned by the caller, who must not touch them until the
 *                   call's work on `stream` has completed
 *
 * The GPU moves the data through the device mapping of the host buffers, so
 * scattered blocks need no staging.  A block index outside the pool skips its
 * slot.  PKV_EINVAL for memory that is not pinned host memory.
 */
pkv_status paged_kv_swap_out(const void* k_cache, const void* v_cache, const pkv_layout* layout,
                             const int32_t* blocks, int32_t n, void* host_k, void* host_v, void* stream);
pkv_status paged_kv_swap_in(void* k_cache, void* v_cache, const pkv_layout* layout, const int32_t* blocks,
                            int32_t n, const void* host_k, const void* host_v, void* stream);

/*
 * Chunked prefill ("How a serving engine actually works", paperfordummies.in,
 * section "Prefill and decode are two different jobs": a long prompt is
 * processed one chunk per step; "Paged Attention and the Block Manager",
 * snowch.github.io ch08, "The build": the host grows the table by the blocks
 * n new tokens need).  Rows of several sequences are packed: sequence s owns
 * rows cu[s] .. cu[s+1]-1 of a [total][heads][head_dim] array (cu[0] = 0,
 * non-decreasing, total = cu[num_seqs]).
 */

/*
 * paged_kv_append_tokens -- the n-token append.  For every s and every row
 * x in [cu_new[s], cu_new[s+1]):
 *     k_cache[slot(s, start_pos[s] + x - cu_new[s])] = k_new[x]   (and v)
 * a bit-exact copy.  Nothing else in the caches changes.
 *
 *   k_new, v_new  [total_new][n_kv_heads][head_dim], element type layout->dtype
 *   cu_new        [num_seqs + 1] int32 device array; total_new = cu_new[num_seqs]
 *                 (passed by value too, to size the grid)
 *   start_pos     [num_seqs] int32: position of each sequence's first new row
 *   other arguments as for paged_kv_append (any block_size)
 *
 * Preconditions: target slots pairwise distinct; the table covers every
 * position.  A row whose position or block lies outside its range is skipped.
 */
pkv_status paged_kv_append_tokens(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const pkv_layout* layout, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* cu_new, const int32_t* start_pos, int32_t num_seqs,
                                  int32_t total_new, void* stream);

/*
 * paged_attention_prefill -- attention of a chunk's queries.  Sequence s holds
 * L = context_lens[s] tokens in the cache, its chunk's n = cu_q[s+1] - cu_q[s]
 * included as the last n (append them first).  Query row cu_q[s] + j sits at
 * position L - n + j and attends to positions 0 .. L - n + j (the earlier
 * context and the chunk up to itself); for query head h, KV head
 * g = h / (n_q_heads / n_kv_heads):
 *     out[cu_q[s] + j][h] = sum_{i <= L-n+j} softmax_i(scale * <q[cu_q[s]+j][h], K_i>) V_i
 * accumulated in fp32, rounded to the cache dtype (round to nearest even).
 * n = 1 gives the same value as paged_attention_decode.
 *
 *   q, out        [total][n_q_heads][head_dim], element type layout->dtype
 *   cu_q          [num_seqs + 1] int32 device array
 *   context_lens  [num_seqs] int32: n <= L <= max_blocks_per_seq * block_size
 *   max_q_len     host int: the longest chunk (sizes the grid); a longer
 *                 chunk gets the rows of its first max_q_len tokens, the rest
 *                 of out is left as it was
 *
 * Supported: fp16 / bf16 caches, block_size 8, 16, 32 or 64, head_dim 64 or
 * 128, group 1, 2, 4 or 8, num_seqs <= 65535, max_q_len x group <= 65535 x 128 query
 * rows, num_seqs x ceil(max_q_len x group / 128) < 2^31 and n_kv_heads x
 * num_seqs < 2^23 (PKV_ENOTSUP otherwise; fp32 prefill is not served).  A sequence whose
 * chunk is empty or longer than its context is skipped.
 * pkv_validate_prefill() checks cu_q, the lengths and the tables on the host.
 */
pkv_status paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* layout,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                                   int32_t n_q_heads, float scale, void* out, void* stream);

/*
 * paged_kv_copy_blocks -- the data half of copy-on-write.
 *
 * A sequence about to write into a block that other sequences also hold takes
 * a private block first, and the tokens the shared block already holds for it
 * (its first n rows) must be in the private block before the write ("How a
 * serving engine actually works", paperfordummies.in, section "Copy-on-write,
 * because you have used fork()"; there the simulation counts the copy but moves
 * no data).  For every i < n_copies:
 *     rows [0, n_rows[i]) of block dst_blocks[i] = the same rows of block src_blocks[i]
 * in both caches, all heads, a bit-exact copy.  Rows >= n_rows[i] of the target
 * and every other block are left as they were.  n_rows[i] = block_size copies a
 * whole block (a beam or a swapped-in sequence); 0 copies nothing.
 *
 *   k_cache, v_cache  the layer's caches (see top of file), changed in place
 *   layout            host pointer; any block_size (the copy does not depend on it)
 *   src_blocks, dst_blocks, n_rows  [n_copies] int32 device arrays
 *
 * Preconditions: the targets of copies with n_rows > 0 are pairwise distinct
 * and none of them is also a source in the same call (a target is a freshly
 * allocated private block); otherwise the result is unspecified.  A copy with a
 * block outside [0, num_blocks) or n_rows outside [0, block_size] is skipped.
 * pkv_validate_copies() checks all of this on host copies of the arrays.
 */
pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const pkv_layout* layout,
                                const int32_t* src_blocks, const int32_t* dst_blocks, const int32_t* n_rows,
                                int32_t n_copies, void* stream);

/*
 * paged_attention_decode -- one decode step of attention through block tables.
 *
 *   q             [num_seqs][n_q_heads][head_dim], element type layout->dtype
 *   k_cache, v_cache, layout, block_tables, max_blocks_per_seq  as above
 *   context_lens  [num_seqs] int32: tokens attended (0 <= L <= max_blocks_per_seq * B)
 *   n_q_heads     a multiple of layout->n_kv_heads
 *   scale         multiplies every score (usually 1 / sqrt(head_dim))
 *   out           [num_seqs][n_q_heads][head_dim], element type layout->dtype
 *
 * Work is split so that every wave of the GPU streams the same number of
 * 16-token tiles whatever the mix of context lengths (the "flat" schedule):
 * a sequence may be cut into several pieces whose partial softmax states
 * (running max, sum of exponentials, unnormalised weighted sum of values) are
 * combined by the log-sum-exp rule.  A fixed partition length can be asked
 * for instead (pkv_set_partition_tokens, or paged_attention_decode_ws).  The
 * split-K workspace is owned by the library (one per device, grown on demand
 * with hipMalloc, freed at unload); callers that must not allocate use
 * paged_attention_decode_ws.  Calls that share the library workspace must be
 * ordered (same stream, or synchronised).
 */
pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const pkv_layout* layout, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                  void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory during the call: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, schedule and output bits as paged_attention_decode; the split-K
 * workspace is a fixed array of PKV_NOALLOC_SCRATCH_BYTES in the library's
 * device code, one per GPU, held from the library's first use on that GPU
 * until the process ends.  The call makes no hipMalloc / hipFree.
 *
 * A batch whose workspace (paged_attention_workspace_size(..., 0)) exceeds
 * PKV_NOALLOC_SCRATCH_BYTES is rejected with PKV_EINVAL.  Every call on one GPU
 * uses that GPU's one array: calls that may overlap on one GPU (different
 * streams, or other threads) race and must be ordered by the caller.  The
 * array keeps the last call's contents; nothing in it needs clearing.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pkv_status paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const pkv_layout* layout, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                          void* stream);

/*
 * Bytes of split-K workspace paged_attention_decode_ws needs for these sizes
 * with partition length part_tokens (0 = the library's choice).  Returns 0 for
 * invalid sizes.  The size is a function of the table width, not of the
 * lengths in a batch: fixed partitions need one record per partition of the
 * longest context a table row can describe (max_blocks_per_seq * block_size
 * tokens), and the flat schedule's records depend on the batch and grid sizes
 * only.  So one workspace sized here serves every batch of these dimensions.
 */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t n_q_heads,
                                      int32_t max_blocks_per_seq, const pkv_layout* layout,
                                      int32_t part_tokens);

/*
 * paged_attention_decode_ws -- paged_attention_decode with an explicit
 * partition length and a caller-owned workspace.
 *
 *   part_tokens  0 for the library's choice (the flat schedule, unless a
 *                different default was set with pkv_set_partition_tokens), or
 *                a fixed partition length: a positive multiple of 16 and of
 *                layout->block_size; each P-token partition of a sequence is
 *                one wave's work and the partitions are merged by the
 *                log-sum-exp rule
 *   workspace    device buffer of at least
 *                paged_attention_workspace_size(..., part_tokens) bytes,
 *                256-byte aligned; may be NULL when that size is 0
 *
 * Runs two kernels: the partition pass (paged_attention_partitions) and, for
 * sequences with more than one partition, the merge (paged_attention_merge).
 */
pkv_status paged_attention_decode_ws(const void* q, const void* k_cache, const void* v_cache,
                                     const pkv_layout* layout, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                     int32_t part_tokens, void* workspace, size_t ws_bytes,
                                     void* stream);

/*
 * The two passes of paged_attention_decode_ws, callable separately (same
 * arguments; the merge must follow the partition pass on the same workspace).
 * The partition pass writes `out` directly for every (sequence, KV head) that
 * one wave (flat schedule) or one partition (fixed partitions) covers whole,
 * and the per-piece softmax state (running max, sum of exponentials,
 * unnormalised weighted sum of values) to the workspace for the others; the
 * merge pass combines those states,
 *     M = max_j m_j,   out = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j,
 * and writes their rows of `out` (and the zero rows of empty sequences under
 * the flat schedule).  The workspace layout is internal.
 */
pkv_status paged_attention_partitions(const void* q, const void* k_cache, const void* v_cache,
                                      const pkv_layout* layout, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                      int32_t part_tokens, void* workspace, size_t ws_bytes,
                                      void* stream);

pkv_status paged_attention_merge(const pkv_layout* layout, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                 void* out, int32_t part_tokens, const void* workspace,
                                 size_t ws_bytes, void* stream);

/*
 * paged_kv_append_attention_decode_ws -- paged_kv_append followed by
 * paged_attention_decode_ws, as one call with the same result: the same
 * caches afterwards (each new row bit-copied to its slot) and the same
 * output bits.  The new token's K/V enter the attention exactly as the
 * append would have stored them ("How a serving engine actually works",
 * paperfordummies.in, "The one formula"; the appended token is attended in
 * the same step -- henryhe.ai, "What's deliberately still missing").
 *
 *   k_new, v_new, positions   as for paged_kv_append
 *   the rest                  as for paged_attention_decode_ws
 *
 * Under the flat schedule this runs two kernels, not three: the decode pass
 * reads the row at positions[s] from k_new / v_new instead of the cache, and
 * the merge pass, after every read of the step, writes the rows to their
 * slots.  Under fixed partitions it is the two calls.  The caches are written
 * during the call (k_cache, v_cache are not const).  Errors as for the two
 * calls; a NULL k_new, v_new or positions is PKV_EINVAL.
 */
pkv_status paged_kv_append_attention_decode_ws(const void* k_new, const void* v_new, const int32_t* positions,
                                               const void* q, void* k_cache, void* v_cache,
                                               const pkv_layout* layout, const int32_t* block_tables,
                                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                                               int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                               int32_t part_tokens, void* workspace, size_t ws_bytes,
                                               void* stream);

/* The same with the library's workspace and partition choice (as paged_attention_decode). */
pkv_status paged_kv_append_attention_decode(const void* k_new, const void* v_new, const int32_t* positions,
                                            const void* q, void* k_cache, void* v_cache, const pkv_layout* layout,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                            float scale, void* out, void* stream);

/*
 * Process-wide partition length used when a call passes 0 (and by
 * paged_attention_decode): a positive multiple of 16, or 0 to restore the
 * library's choice (the flat schedule; batches of more than 8000 sequences,
 * or with more than 2^30 tiles, use 512-token partitions).  Returns
 * PKV_EINVAL otherwise.  A call whose block size is larger than this length,
 * or does not divide it, uses the next multiple of the block size (a length
 * of 16 with 64-token blocks partitions by 64).
 */
pkv_status pkv_set_partition_tokens(int32_t tokens);

/* Partition length the library would use for these sizes (0 = flat schedule). */
int32_t pkv_partition_tokens_for(int32_t num_seqs, int32_t n_q_heads, int32_t max_blocks_per_seq,
                                 const pkv_layout* layout);

/*
 * pkv_validate -- host-side debugging check of a step's bookkeeping (no GPU
 * work).  All pointers are HOST pointers.  Checks that every table entry a
 * sequence uses (its first ceil(L / B) entries, L = context_lens[s]) lies in
 * [0, num_blocks), that 0 <= L <= max_blocks_per_seq * B, and, when positions
 * is non-NULL, that every append slot lies inside the sequence's blocks and
 * that no two sequences append to the same slot.  Returns PKV_OK, PKV_EOOB
 * (range) or PKV_EINVAL (shape, or duplicate append slots) with a message.
 */
pkv_status pkv_validate(const pkv_layout* layout, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* positions, int32_t num_seqs);

/*
 * pkv_validate_copies -- host-side check of a paged_kv_copy_blocks batch (HOST
 * pointers, no GPU work): blocks inside the pool and row counts inside
 * [0, block_size] (else PKV_EOOB), and the targets of non-empty copies pairwise
 * distinct and disjoint from the sources (else PKV_EINVAL), with a message.
 */
pkv_status pkv_validate_copies(const pkv_layout* layout, const int32_t* src_blocks, const int32_t* dst_blocks,
                               const int32_t* n_rows, int32_t n_copies);

/*
 * pkv_validate_prefill -- host-side check of a prefill step (HOST pointers):
 * cu_q starts at 0 and never decreases, every chunk fits max_q_len and its
 * context (n <= L <= max_blocks_per_seq * block_size), and every table entry
 * the context uses lies in the pool.  PKV_OK, PKV_EINVAL or PKV_EOOB.
 */
pkv_status pkv_validate_prefill(const pkv_layout* layout, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* cu_q, const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_q_len);

/* Message of this thread's last non-OK call ("" if none).  Owned by the library. */
const char* pkv_last_error(void);

/* Library version string, e.g. "pagedkv 0.1 gfx950". */
const char* pkv_version(void);

/*
 * Measurement helpers (not part of the decode path):
 *   pkv_probe_read  -- streams `bytes` (a multiple of 16) from `src` with
 *                      16-byte loads and writes one checksum word per
 *                      workgroup to `sink` (>= 4096 floats); gives the
 *                      achievable HBM read rate;
 *   pkv_probe_copy  -- copies `bytes` (a multiple of 16) from src to dst; a
 *                      plain kernel of known traffic for calibrating counters.
 */
pkv_status pkv_probe_read(const void* src, size_t bytes, float* sink, void* stream);
pkv_status pkv_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
