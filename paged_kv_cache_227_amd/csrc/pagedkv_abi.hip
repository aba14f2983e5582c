// pagedkv_abi.hip -- the C ABI declared in include/pagedkv.h: argument
// checks, dtype / head_dim / group dispatch, split-K planning, the library's
// workspace, status codes and the per-thread error message.  Host code only;
// every step of the path runs in the kernels of append.hip, copy_blocks.hip,
// decode.hip, prefill.hip and swap.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "pagedkv.h"
#include "pkv_launch.h"

namespace {

thread_local std::string g_last_error;
std::atomic<int32_t> g_part_tokens{0};

constexpr int kTileTokens = 16;  // the decode and prefill kernels stream 16-token tiles

// Block sizes the decode and prefill kernels serve: powers of two from 8 to 64
// tokens (a 16-token tile then lies in one block, or in two when B = 8).
int decode_block_shift(int32_t B) {
    switch (B) {
        case 8: return 3;
        case 16: return 4;
        case 32: return 5;
        case 64: return 6;
        default: return -1;
    }
}
constexpr int32_t kDefaultPartTokens = 512;
constexpr int32_t kMinTilesPerWorker = 4;
constexpr size_t kWsAlign = 256;

pkv_status fail(pkv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pkv_status fail(pkv_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

pkv_status ok() {
    return PKV_OK;
}

int elt_bytes(int32_t dtype) {
    return dtype == PKV_F32 ? 4 : (dtype == PKV_F16 || dtype == PKV_BF16) ? 2 : 0;
}

pkv_status check_layout(const pkv_layout* L) {
    if (!L) return fail(PKV_EINVAL, "layout is NULL");
    if (L->num_blocks < 1 || L->block_size < 1 || L->n_kv_heads < 1 || L->head_dim < 1)
        return fail(PKV_EINVAL, "layout sizes must be positive (num_blocks %d, block_size %d, "
                                "n_kv_heads %d, head_dim %d)",
                    L->num_blocks, L->block_size, L->n_kv_heads, L->head_dim);
    if (elt_bytes(L->dtype) == 0) return fail(PKV_EINVAL, "unknown dtype code %d", L->dtype);
    const int64_t row = (int64_t)L->n_kv_heads * L->head_dim * elt_bytes(L->dtype);
    if (row > (1 << 24)) return fail(PKV_EINVAL, "a token row of %lld bytes is too large", (long long)row);
    return PKV_OK;
}

pkv_status hip_fail(hipError_t e, const char* what) {
    return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// The flat schedule serves a batch when its per-workgroup LDS holds the batch
// and its tile count fits comfortably in int32.
bool flat_fits(int32_t num_seqs, int32_t max_blocks, const pkv_layout* L) {
    const int64_t tiles = ((int64_t)max_blocks * L->block_size + kTileTokens - 1) / kTileTokens;
    return num_seqs <= pkv::kMaxFlatSeqs && (int64_t)num_seqs * L->n_kv_heads * tiles <= ((int64_t)1 << 30);
}

// 0 (the library's choice) selects the flat schedule: equal tile ranges per
// wave, whatever the length mix.  Batches it cannot serve use 512-token
// partitions.
pkv_status resolve_partition(int32_t requested, int32_t num_seqs, int32_t max_blocks, const pkv_layout* L,
                             int32_t* out) {
    int32_t P = requested;
    const int32_t unit = std::max<int32_t>(L->block_size, kTileTokens);
    if (P == 0) {
        // the process-wide setting is a multiple of 16; it is rounded up to
        // whole blocks of this layout
        P = g_part_tokens.load();
        P = (P + unit - 1) / unit * unit;
    }
    if (P < 0 || P % unit != 0)
        return fail(PKV_EINVAL, "partition length %d is not a positive multiple of %d (the block size and 16)", P,
                    unit);
    if (P == 0 && !flat_fits(num_seqs, max_blocks, L)) P = kDefaultPartTokens;
    *out = P;
    return PKV_OK;
}

struct Plan {
    int32_t part_tokens;  // 0: flat schedule
    int32_t n_parts_max;  // fixed partitions only
    size_t hdr_bytes;     // flat only: the schedule header
    size_t acc_bytes;
    size_t ws_bytes;      // total; 0 when nothing is needed
};

size_t round_up(size_t x) {
    return (x + kWsAlign - 1) / kWsAlign * kWsAlign;
}

Plan make_plan(int32_t num_seqs, int32_t n_q_heads, int32_t max_blocks, const pkv_layout* L, int32_t P) {
    Plan pl{};
    pl.part_tokens = P;
    if (P == 0) {
        // records of NH * G query heads (NH KV heads per wave), indexed by
        // (sequence, head group) + wave: fewer than num_seqs * Hkv / NH + waves
        // of them, so (num_seqs * Hkv + waves * NH) * G head rows at most
        const int G = n_q_heads / L->n_kv_heads;
        const size_t NH = (size_t)pkv::decode_heads_per_wave(L->dtype, L->head_dim, G, L->n_kv_heads);
        const size_t recs = (size_t)num_seqs * L->n_kv_heads + (size_t)pkv::kMaxFlatWorkers * NH;
        pl.n_parts_max = 1;
        pl.hdr_bytes = round_up((size_t)(num_seqs + 4 + pkv::kMaxFlatPeriod) * sizeof(int32_t));
        pl.acc_bytes = round_up(recs * G * L->head_dim * sizeof(float));
        pl.ws_bytes = pl.hdr_bytes + pl.acc_bytes + recs * G * 2 * sizeof(float);
        return pl;
    }
    const int64_t max_tokens = (int64_t)max_blocks * L->block_size;
    pl.n_parts_max = (int32_t)std::max<int64_t>(1, (max_tokens + P - 1) / P);
    if (pl.n_parts_max <= 1) return pl;
    const size_t slots = (size_t)num_seqs * n_q_heads * pl.n_parts_max;
    pl.acc_bytes = round_up(slots * L->head_dim * sizeof(float));
    pl.ws_bytes = pl.acc_bytes + slots * 2 * sizeof(float);
    return pl;
}

pkv_status check_decode(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* L,
                        const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                        int32_t num_seqs, int32_t n_q_heads, float scale, const void* out) {
    pkv_status st = check_layout(L);
    if (st != PKV_OK) return st;
    if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
    if (max_blocks < 1) return fail(PKV_EINVAL, "max_blocks_per_seq %d < 1", max_blocks);
    if (n_q_heads < 1 || n_q_heads % L->n_kv_heads != 0)
        return fail(PKV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads,
                    L->n_kv_heads);
    if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
    if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out))
        return fail(PKV_EINVAL, "a required pointer is NULL");
    if ((int64_t)max_blocks * L->block_size > INT32_MAX)
        return fail(PKV_EINVAL, "max_blocks_per_seq * block_size overflows int32");
    if ((int64_t)num_seqs * n_q_heads > INT32_MAX / 4)
        return fail(PKV_EINVAL, "num_seqs * n_q_heads is too large");
    if (decode_block_shift(L->block_size) < 0)
        return fail(PKV_ENOTSUP, "decode serves block sizes 8, 16, 32 and 64 (got %d)", L->block_size);
    const int group = n_q_heads / L->n_kv_heads;
    if (!pkv::decode_supported(L->dtype, L->head_dim, group))
        return fail(PKV_ENOTSUP, "no kernel for dtype %d, head_dim %d, group %d", L->dtype, L->head_dim,
                    group);
    if (num_seqs > 65535) return fail(PKV_ENOTSUP, "num_seqs %d exceeds 65535", num_seqs);
    if (L->n_kv_heads > 65535) return fail(PKV_ENOTSUP, "n_kv_heads %d exceeds 65535", L->n_kv_heads);
    return PKV_OK;
}

pkv::DecodeParams make_params(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* L,
                              const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                              int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                              const Plan& pl, void* workspace) {
    pkv::DecodeParams p{};
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = out;
    char* ws = static_cast<char*>(workspace);
    p.ws_hdr = ws ? reinterpret_cast<int32_t*>(ws) : nullptr;
    p.ws_acc = ws ? reinterpret_cast<float*>(ws + pl.hdr_bytes) : nullptr;
    p.ws_ml = ws ? reinterpret_cast<float*>(ws + pl.hdr_bytes + pl.acc_bytes) : nullptr;
    p.min_tiles_per_worker = kMinTilesPerWorker;
    p.num_blocks = L->num_blocks;
    p.n_kv_heads = L->n_kv_heads;
    p.n_q_heads = n_q_heads;
    p.max_blocks = max_blocks;
    p.num_seqs = num_seqs;
    p.part_tokens = pl.part_tokens;
    p.n_parts_max = pl.n_parts_max;
    p.block_shift = decode_block_shift(L->block_size);
    p.scale_log2 = scale * 1.4426950408889634f;
    return p;
}

pkv_status check_workspace(const Plan& pl, const void* workspace, size_t ws_bytes) {
    if (pl.ws_bytes == 0) return PKV_OK;
    if (!workspace) return fail(PKV_EINVAL, "workspace is NULL but %zu bytes are needed", pl.ws_bytes);
    if (ws_bytes < pl.ws_bytes)
        return fail(PKV_EINVAL, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, pl.ws_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign != 0)
        return fail(PKV_EINVAL, "workspace is not %zu-byte aligned", kWsAlign);
    return PKV_OK;
}

// The library's own split-K workspace, one per device, grown on demand.
struct DeviceWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

struct WorkspaceReleaser {
    ~WorkspaceReleaser() {
        // Process teardown: the runtime may already be gone, so errors are ignored.
        for (auto& w : g_ws)
            if (w.ptr) (void)hipFree(w.ptr);
    }
} g_ws_releaser;

pkv_status library_workspace(size_t need, void** out) {
    *out = nullptr;
    if (need == 0) return PKV_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
    DeviceWorkspace& w = g_ws[dev];
    if (w.bytes < need) {
        if (w.ptr) {
            e = hipFree(w.ptr);  // synchronises the device: in-flight users finish first
            w.ptr = nullptr;
            w.bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree(workspace)");
        }
        const size_t grown = std::max(need, need + need / 4);
        e = hipMalloc(&w.ptr, grown);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return hip_fail(e, "hipMalloc(workspace)");
        }
        w.bytes = grown;
    }
    *out = w.ptr;
    return PKV_OK;
}

// Split-K workspace for callers that cannot allocate (paged_attention_decode_noalloc):
// one fixed array per device, created with the code object and held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the host
// the name stands for a host-side shadow, not the device array): it passes the
// device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;  // per device; nullptr until looked up

pkv_status device_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const pkv_layout* layout, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* positions, int32_t num_seqs,
                           void* stream) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
    if (max_blocks_per_seq < 1) return fail(PKV_EINVAL, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
    if (num_seqs == 0) return ok();
    if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !positions)
        return fail(PKV_EINVAL, "a required pointer is NULL");
    if (num_seqs > INT32_MAX / 2) return fail(PKV_EINVAL, "num_seqs too large");
    pkv::AppendParams p{};
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.positions = positions;
    p.num_blocks = layout->num_blocks;
    p.block_size = layout->block_size;
    p.max_blocks = max_blocks_per_seq;
    p.num_seqs = num_seqs;
    p.row_bytes = layout->n_kv_heads * layout->head_dim * elt_bytes(layout->dtype);
    hipError_t e = pkv::launch_append(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "append launch");
    return ok();
}

pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const pkv_layout* layout,
                                const int32_t* src_blocks, const int32_t* dst_blocks, const int32_t* n_rows,
                                int32_t n_copies, void* stream) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (n_copies < 0) return fail(PKV_EINVAL, "n_copies %d < 0", n_copies);
    if (n_copies == 0) return ok();
    if (!k_cache || !v_cache || !src_blocks || !dst_blocks || !n_rows)
        return fail(PKV_EINVAL, "a required pointer is NULL");
    pkv::CopyParams p{};
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.src_blocks = src_blocks;
    p.dst_blocks = dst_blocks;
    p.n_rows = n_rows;
    p.num_blocks = layout->num_blocks;
    p.block_size = layout->block_size;
    p.n_copies = n_copies;
    p.row_bytes = (int64_t)layout->n_kv_heads * layout->head_dim * elt_bytes(layout->dtype);
    hipError_t e = pkv::launch_copy_blocks(p, static_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidConfiguration) return fail(PKV_EINVAL, "%d copies exceed the launch grid", n_copies);
    if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
    return ok();
}

pkv_status paged_kv_append_tokens(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const pkv_layout* layout, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* cu_new, const int32_t* start_pos, int32_t num_seqs,
                                  int32_t total_new, void* stream) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || total_new < 0)
        return fail(PKV_EINVAL, "num_seqs %d or total_new %d < 0", num_seqs, total_new);
    if (max_blocks_per_seq < 1) return fail(PKV_EINVAL, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
    if (num_seqs == 0 || total_new == 0) return ok();
    if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !cu_new || !start_pos)
        return fail(PKV_EINVAL, "a required pointer is NULL");
    pkv::AppendTokensParams p{};
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.cu_new = cu_new;
    p.start_pos = start_pos;
    p.num_blocks = layout->num_blocks;
    p.block_size = layout->block_size;
    p.max_blocks = max_blocks_per_seq;
    p.num_seqs = num_seqs;
    p.total = total_new;
    p.row_bytes = layout->n_kv_heads * layout->head_dim * elt_bytes(layout->dtype);
    hipError_t e = pkv::launch_append_tokens(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "append_tokens launch");
    return ok();
}

pkv_status paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* layout,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len,
                                   int32_t n_q_heads, float scale, void* out, void* stream) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || max_q_len < 0) return fail(PKV_EINVAL, "num_seqs %d or max_q_len %d < 0", num_seqs, max_q_len);
    if (max_blocks_per_seq < 1) return fail(PKV_EINVAL, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
    if (n_q_heads < 1 || n_q_heads % layout->n_kv_heads != 0)
        return fail(PKV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads,
                    layout->n_kv_heads);
    if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
    if ((int64_t)max_blocks_per_seq * layout->block_size > INT32_MAX)
        return fail(PKV_EINVAL, "max_blocks_per_seq * block_size overflows int32");
    if (num_seqs > 0 && max_q_len > 0 && (!q || !k_cache || !v_cache || !block_tables || !cu_q || !context_lens || !out))
        return fail(PKV_EINVAL, "a required pointer is NULL");
    if (decode_block_shift(layout->block_size) < 0)
        return fail(PKV_ENOTSUP, "prefill serves block sizes 8, 16, 32 and 64 (got %d)", layout->block_size);
    const int group = n_q_heads / layout->n_kv_heads;
    if (!pkv::prefill_supported(layout->dtype, layout->head_dim, group))
        return fail(PKV_ENOTSUP, "no prefill kernel for dtype %d, head_dim %d, group %d (16-bit caches only)",
                    layout->dtype, layout->head_dim, group);
    if (num_seqs > 65535) return fail(PKV_ENOTSUP, "num_seqs %d exceeds 65535", num_seqs);
    if ((int64_t)max_q_len * group > pkv::kMaxPrefillTiles * pkv::kPrefillRows)
        return fail(PKV_ENOTSUP, "max_q_len %d x group %d exceeds %lld query rows", max_q_len, group,
                    (long long)(pkv::kMaxPrefillTiles * pkv::kPrefillRows));
    if (num_seqs == 0 || max_q_len == 0) return ok();
    {
        // the grid: (KV heads x sequences, tiles), 512 threads per workgroup
        const int64_t tiles = ((int64_t)max_q_len * group + pkv::kPrefillRows - 1) / pkv::kPrefillRows;
        if (tiles * num_seqs > INT32_MAX || (int64_t)layout->n_kv_heads * num_seqs * 512 > UINT32_MAX)
            return fail(PKV_ENOTSUP, "prefill grid too large: %d sequences x %lld tiles x %d KV heads", num_seqs,
                        (long long)tiles, layout->n_kv_heads);
    }
    pkv::PrefillParams p{};
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.cu_q = cu_q;
    p.context_lens = context_lens;
    p.out = out;
    p.num_blocks = layout->num_blocks;
    p.n_kv_heads = layout->n_kv_heads;
    p.n_q_heads = n_q_heads;
    p.max_blocks = max_blocks_per_seq;
    p.num_seqs = num_seqs;
    p.max_q_len = max_q_len;
    p.block_shift = decode_block_shift(layout->block_size);
    p.scale_log2 = scale * 1.4426950408889634f;
    hipError_t e = pkv::launch_prefill(p, layout->dtype, layout->head_dim, group, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

namespace {

// Device view of a pinned host buffer, or an error for memory that is not.
pkv_status device_view_of_host(const void* host, void** dev, const char* name) {
    hipError_t e = hipHostGetDevicePointer(dev, const_cast<void*>(host), 0);
    if (e != hipSuccess || !*dev) {
        (void)hipGetLastError();  // clear the sticky error of the failed lookup
        return fail(PKV_EINVAL, "%s is not pinned host memory (allocate it with hipHostMalloc)", name);
    }
    return PKV_OK;
}

pkv_status swap_common(void* k_cache, void* v_cache, const pkv_layout* layout, const int32_t* blocks, int32_t n,
                       const void* host_k, const void* host_v, bool to_cache, void* stream) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (n < 0) return fail(PKV_EINVAL, "n %d < 0", n);
    if (n == 0) return ok();
    if (!k_cache || !v_cache || !blocks || !host_k || !host_v) return fail(PKV_EINVAL, "a required pointer is NULL");
    const int64_t blk_bytes =
        (int64_t)layout->block_size * layout->n_kv_heads * layout->head_dim * elt_bytes(layout->dtype);
    if (blk_bytes % 16 != 0) return fail(PKV_ENOTSUP, "a block of %lld bytes is not a multiple of 16", (long long)blk_bytes);
    pkv::SwapParams p{};
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.blocks = blocks;
    st = device_view_of_host(host_k, &p.host_k, "host_k");
    if (st != PKV_OK) return st;
    st = device_view_of_host(host_v, &p.host_v, "host_v");
    if (st != PKV_OK) return st;
    p.num_blocks = layout->num_blocks;
    p.n = n;
    p.blk_bytes = blk_bytes;
    hipError_t e = pkv::launch_swap(p, to_cache, static_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidConfiguration) return fail(PKV_EINVAL, "%d blocks exceed the launch grid", n);
    if (e != hipSuccess) return hip_fail(e, "swap launch");
    return ok();
}

}  // namespace

pkv_status paged_kv_swap_out(const void* k_cache, const void* v_cache, const pkv_layout* layout,
                             const int32_t* blocks, int32_t n, void* host_k, void* host_v, void* stream) {
    return swap_common(const_cast<void*>(k_cache), const_cast<void*>(v_cache), layout, blocks, n, host_k, host_v,
                       false, stream);
}

pkv_status paged_kv_swap_in(void* k_cache, void* v_cache, const pkv_layout* layout, const int32_t* blocks,
                            int32_t n, const void* host_k, const void* host_v, void* stream) {
    return swap_common(k_cache, v_cache, layout, blocks, n, host_k, host_v, true, stream);
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t n_q_heads, int32_t max_blocks_per_seq,
                                      const pkv_layout* layout, int32_t part_tokens) {
    if (check_layout(layout) != PKV_OK || num_seqs < 0 || n_q_heads < 1 || max_blocks_per_seq < 1) return 0;
    int32_t P = 0;
    if (resolve_partition(part_tokens, num_seqs, max_blocks_per_seq, layout, &P) != PKV_OK)
        return 0;
    return make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, P).ws_bytes;
}

pkv_status paged_attention_partitions(const void* q, const void* k_cache, const void* v_cache,
                                      const pkv_layout* layout, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                      int32_t part_tokens, void* workspace, size_t ws_bytes, void* stream) {
    pkv_status st = check_decode(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                 context_lens, num_seqs, n_q_heads, scale, out);
    if (st != PKV_OK) return st;
    int32_t P = 0;
    st = resolve_partition(part_tokens, num_seqs, max_blocks_per_seq, layout, &P);
    if (st != PKV_OK) return st;
    const Plan pl = make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, P);
    st = check_workspace(pl, workspace, ws_bytes);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return ok();
    if ((int64_t)pl.n_parts_max * num_seqs > 0x7fffffff)
        return fail(PKV_ENOTSUP, "%d partitions per sequence x %d sequences exceed the launch grid", pl.n_parts_max,
                    num_seqs);
    const pkv::DecodeParams p = make_params(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                            context_lens, num_seqs, n_q_heads, scale, out, pl, workspace);
    hipError_t e = pkv::launch_decode_partitions(p, layout->dtype, layout->head_dim,
                                                 n_q_heads / layout->n_kv_heads,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "partition launch");
    return ok();
}

pkv_status paged_attention_merge(const pkv_layout* layout, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads, void* out,
                                 int32_t part_tokens, const void* workspace, size_t ws_bytes, void* stream) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || max_blocks_per_seq < 1 || n_q_heads < 1 || n_q_heads % layout->n_kv_heads != 0)
        return fail(PKV_EINVAL, "bad sizes (num_seqs %d, max_blocks_per_seq %d, n_q_heads %d)", num_seqs,
                    max_blocks_per_seq, n_q_heads);
    if (num_seqs > 0 && (!context_lens || !out)) return fail(PKV_EINVAL, "a required pointer is NULL");
    if (decode_block_shift(layout->block_size) < 0)
        return fail(PKV_ENOTSUP, "decode serves block sizes 8, 16, 32 and 64 (got %d)", layout->block_size);
    if (!pkv::decode_supported(layout->dtype, layout->head_dim, n_q_heads / layout->n_kv_heads))
        return fail(PKV_ENOTSUP, "no kernel for dtype %d, head_dim %d", layout->dtype, layout->head_dim);
    int32_t P = 0;
    st = resolve_partition(part_tokens, num_seqs, max_blocks_per_seq, layout, &P);
    if (st != PKV_OK) return st;
    const Plan pl = make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, P);
    st = check_workspace(pl, workspace, ws_bytes);
    if (st != PKV_OK) return st;
    // Fixed partitions: nothing to merge when no sequence can span two.  The flat
    // schedule always runs its merge pass (split pairs, and zeros for L = 0).
    if (num_seqs == 0 || (pl.part_tokens > 0 && pl.n_parts_max <= 1)) return ok();
    const pkv::DecodeParams p = make_params(nullptr, nullptr, nullptr, layout, nullptr, max_blocks_per_seq,
                                            context_lens, num_seqs, n_q_heads, 1.f, out, pl,
                                            const_cast<void*>(workspace));
    hipError_t e = pkv::launch_decode_merge(p, layout->dtype, layout->head_dim, n_q_heads / layout->n_kv_heads,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return ok();
}

pkv_status paged_attention_decode_ws(const void* q, const void* k_cache, const void* v_cache,
                                     const pkv_layout* layout, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                     int32_t n_q_heads, float scale, void* out, int32_t part_tokens,
                                     void* workspace, size_t ws_bytes, void* stream) {
    pkv_status st = paged_attention_partitions(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                               context_lens, num_seqs, n_q_heads, scale, out, part_tokens,
                                               workspace, ws_bytes, stream);
    if (st != PKV_OK) return st;
    return paged_attention_merge(layout, max_blocks_per_seq, context_lens, num_seqs, n_q_heads, out,
                                 part_tokens, workspace, ws_bytes, stream);
}

pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const pkv_layout* layout, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t n_q_heads, float scale, void* out, void* stream) {
    pkv_status st = check_decode(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                 context_lens, num_seqs, n_q_heads, scale, out);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return ok();
    int32_t P = 0;
    st = resolve_partition(0, num_seqs, max_blocks_per_seq, layout, &P);
    if (st != PKV_OK) return st;
    const Plan pl = make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, P);
    void* ws = nullptr;
    st = library_workspace(pl.ws_bytes, &ws);
    if (st != PKV_OK) return st;
    return paged_attention_decode_ws(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                     context_lens, num_seqs, n_q_heads, scale, out, P, ws, pl.ws_bytes,
                                     stream);
}

pkv_status paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const pkv_layout* layout, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                          int32_t n_q_heads, float scale, void* out, void* stream) {
    pkv_status st = check_decode(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                 context_lens, num_seqs, n_q_heads, scale, out);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return ok();
    int32_t P = 0;
    st = resolve_partition(0, num_seqs, max_blocks_per_seq, layout, &P);
    if (st != PKV_OK) return st;
    const Plan pl = make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, P);
    if (pl.ws_bytes > kScratchBytes)
        return fail(PKV_EINVAL,
                    "this batch needs %zu bytes of split-K workspace; the no-allocation call holds %zu "
                    "(use paged_attention_decode_ws with a workspace of that size)",
                    pl.ws_bytes, kScratchBytes);
    void* ws = nullptr;
    st = device_scratch(&ws);
    if (st != PKV_OK) return st;
    // Nothing in the workspace needs to start at zero: the partition pass writes
    // the schedule header and every record before the merge pass reads them.
    return paged_attention_decode_ws(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq, context_lens,
                                     num_seqs, n_q_heads, scale, out, P, ws, kScratchBytes, stream);
}

pkv_status paged_kv_append_attention_decode_ws(const void* k_new, const void* v_new, const int32_t* positions,
                                               const void* q, void* k_cache, void* v_cache,
                                               const pkv_layout* layout, const int32_t* block_tables,
                                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                                               int32_t num_seqs, int32_t n_q_heads, float scale, void* out,
                                               int32_t part_tokens, void* workspace, size_t ws_bytes,
                                               void* stream) {
    pkv_status st = check_decode(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq, context_lens,
                                 num_seqs, n_q_heads, scale, out);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return ok();
    if (!k_new || !v_new || !positions) return fail(PKV_EINVAL, "a required pointer is NULL");
    int32_t P = 0;
    st = resolve_partition(part_tokens, num_seqs, max_blocks_per_seq, layout, &P);
    if (st != PKV_OK) return st;
    if (P > 0) {  // fixed partitions: the two calls
        st = paged_kv_append(k_new, v_new, k_cache, v_cache, layout, block_tables, max_blocks_per_seq, positions,
                             num_seqs, stream);
        if (st != PKV_OK) return st;
        return paged_attention_decode_ws(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq,
                                         context_lens, num_seqs, n_q_heads, scale, out, P, workspace, ws_bytes,
                                         stream);
    }
    const Plan pl = make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, 0);
    st = check_workspace(pl, workspace, ws_bytes);
    if (st != PKV_OK) return st;
    pkv::DecodeParams p = make_params(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq, context_lens,
                                      num_seqs, n_q_heads, scale, out, pl, workspace);
    p.k_new = k_new;
    p.v_new = v_new;
    p.positions = positions;
    p.k_cache_w = k_cache;
    p.v_cache_w = v_cache;
    const int group = n_q_heads / layout->n_kv_heads;
    hipError_t e = pkv::launch_decode_partitions(p, layout->dtype, layout->head_dim, group,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "partition launch");
    e = pkv::launch_decode_merge(p, layout->dtype, layout->head_dim, group, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return ok();
}

pkv_status paged_kv_append_attention_decode(const void* k_new, const void* v_new, const int32_t* positions,
                                            const void* q, void* k_cache, void* v_cache, const pkv_layout* layout,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                            float scale, void* out, void* stream) {
    pkv_status st = check_decode(q, k_cache, v_cache, layout, block_tables, max_blocks_per_seq, context_lens,
                                 num_seqs, n_q_heads, scale, out);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return ok();
    if (!k_new || !v_new || !positions) return fail(PKV_EINVAL, "a required pointer is NULL");
    int32_t P = 0;
    st = resolve_partition(0, num_seqs, max_blocks_per_seq, layout, &P);
    if (st != PKV_OK) return st;
    const Plan pl = make_plan(num_seqs, n_q_heads, max_blocks_per_seq, layout, P);
    void* ws = nullptr;
    st = library_workspace(pl.ws_bytes, &ws);
    if (st != PKV_OK) return st;
    return paged_kv_append_attention_decode_ws(k_new, v_new, positions, q, k_cache, v_cache, layout, block_tables,
                                               max_blocks_per_seq, context_lens, num_seqs, n_q_heads, scale, out, P,
                                               ws, pl.ws_bytes, stream);
}

pkv_status pkv_set_partition_tokens(int32_t tokens) {
    if (tokens < 0 || tokens % kTileTokens != 0)
        return fail(PKV_EINVAL, "partition length %d is not 0 or a positive multiple of %d", tokens,
                    kTileTokens);
    g_part_tokens.store(tokens);
    return PKV_OK;
}

int32_t pkv_partition_tokens_for(int32_t num_seqs, int32_t n_q_heads, int32_t max_blocks_per_seq,
                                 const pkv_layout* layout) {
    if (check_layout(layout) != PKV_OK) return 0;
    int32_t P = 0;
    if (resolve_partition(0, num_seqs, max_blocks_per_seq, layout, &P) != PKV_OK) return 0;
    return P;
}

pkv_status pkv_validate(const pkv_layout* layout, const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, const int32_t* positions, int32_t num_seqs) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || max_blocks_per_seq < 1) return fail(PKV_EINVAL, "bad num_seqs or max_blocks_per_seq");
    if (num_seqs > 0 && (!block_tables || !context_lens)) return fail(PKV_EINVAL, "a required pointer is NULL");
    const int64_t B = layout->block_size;
    std::vector<int64_t> slots;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
        const int64_t L = context_lens[s];
        if (L < 0 || L > (int64_t)max_blocks_per_seq * B)
            return fail(PKV_EOOB, "sequence %d: context length %lld outside [0, %lld]", s, (long long)L,
                        (long long)max_blocks_per_seq * B);
        const int64_t nb = (L + B - 1) / B;
        for (int64_t b = 0; b < nb; ++b)
            if (row[b] < 0 || row[b] >= layout->num_blocks)
                return fail(PKV_EOOB, "sequence %d: table entry %lld = %d outside [0, %d)", s, (long long)b,
                            row[b], layout->num_blocks);
        if (positions) {
            const int64_t p = positions[s];
            if (p < 0 || p / B >= max_blocks_per_seq)
                return fail(PKV_EOOB, "sequence %d: position %lld outside the table", s, (long long)p);
            const int32_t blk = row[p / B];
            if (blk < 0 || blk >= layout->num_blocks)
                return fail(PKV_EOOB, "sequence %d: position %lld maps to block %d outside [0, %d)", s,
                            (long long)p, blk, layout->num_blocks);
            slots.push_back((int64_t)blk * B + p % B);
        }
    }
    if (!slots.empty()) {
        std::vector<int64_t> sorted = slots;
        std::sort(sorted.begin(), sorted.end());
        for (size_t i = 1; i < sorted.size(); ++i)
            if (sorted[i] == sorted[i - 1])
                return fail(PKV_EINVAL, "two sequences append to slot %lld", (long long)sorted[i]);
    }
    return PKV_OK;
}

pkv_status pkv_validate_prefill(const pkv_layout* layout, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* cu_q, const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_q_len) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || max_blocks_per_seq < 1) return fail(PKV_EINVAL, "bad num_seqs or max_blocks_per_seq");
    if (num_seqs > 0 && (!block_tables || !cu_q || !context_lens)) return fail(PKV_EINVAL, "a required pointer is NULL");
    if (num_seqs > 0 && cu_q[0] != 0) return fail(PKV_EINVAL, "cu_q[0] = %d, not 0", cu_q[0]);
    const int64_t B = layout->block_size;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t n = (int64_t)cu_q[s + 1] - cu_q[s];
        const int64_t L = context_lens[s];
        if (n < 0) return fail(PKV_EINVAL, "cu_q decreases at sequence %d", s);
        if (n > max_q_len) return fail(PKV_EINVAL, "sequence %d: chunk of %lld tokens > max_q_len %d", s, (long long)n, max_q_len);
        if (L < n || L > (int64_t)max_blocks_per_seq * B)
            return fail(PKV_EOOB, "sequence %d: context length %lld outside [%lld, %lld]", s, (long long)L,
                        (long long)n, (long long)max_blocks_per_seq * B);
        const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int64_t b = 0; b < (L + B - 1) / B; ++b)
            if (row[b] < 0 || row[b] >= layout->num_blocks)
                return fail(PKV_EOOB, "sequence %d: table entry %lld = %d outside [0, %d)", s, (long long)b, row[b],
                            layout->num_blocks);
    }
    return PKV_OK;
}

pkv_status pkv_validate_copies(const pkv_layout* layout, const int32_t* src_blocks, const int32_t* dst_blocks,
                               const int32_t* n_rows, int32_t n_copies) {
    pkv_status st = check_layout(layout);
    if (st != PKV_OK) return st;
    if (n_copies < 0) return fail(PKV_EINVAL, "n_copies %d < 0", n_copies);
    if (n_copies > 0 && (!src_blocks || !dst_blocks || !n_rows)) return fail(PKV_EINVAL, "a required pointer is NULL");
    std::vector<int32_t> dsts, srcs;
    for (int32_t i = 0; i < n_copies; ++i) {
        if (src_blocks[i] < 0 || src_blocks[i] >= layout->num_blocks || dst_blocks[i] < 0 ||
            dst_blocks[i] >= layout->num_blocks)
            return fail(PKV_EOOB, "copy %d: block %d -> %d outside [0, %d)", i, src_blocks[i], dst_blocks[i],
                        layout->num_blocks);
        if (n_rows[i] < 0 || n_rows[i] > layout->block_size)
            return fail(PKV_EOOB, "copy %d: %d rows outside [0, %d]", i, n_rows[i], layout->block_size);
        if (n_rows[i] == 0) continue;  // moves nothing, so overlaps nothing
        dsts.push_back(dst_blocks[i]);
        srcs.push_back(src_blocks[i]);
    }
    std::sort(dsts.begin(), dsts.end());
    std::sort(srcs.begin(), srcs.end());
    for (size_t i = 1; i < dsts.size(); ++i)
        if (dsts[i] == dsts[i - 1]) return fail(PKV_EINVAL, "two copies write block %d", dsts[i]);
    for (int32_t d : dsts)
        if (std::binary_search(srcs.begin(), srcs.end(), d))
            return fail(PKV_EINVAL, "block %d is both a copy's source and a copy's target", d);
    return PKV_OK;
}

const char* pkv_last_error(void) {
    return g_last_error.c_str();
}

const char* pkv_version(void) {
    return "pagedkv 0.1 gfx950";
}

pkv_status pkv_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || bytes % 16 != 0) return fail(PKV_EINVAL, "probe_read: NULL pointer or size not a multiple of 16");
    hipError_t e = pkv::launch_probe_read(src, bytes, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "probe_read launch");
    return PKV_OK;
}

pkv_status pkv_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 != 0) return fail(PKV_EINVAL, "probe_copy: NULL pointer or size not a multiple of 16");
    hipError_t e = pkv::launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "probe_copy launch");
    return PKV_OK;
}

}  // extern "C"
