// prefill.hip -- chunked prefill on gfx950: the n-token append and the
// attention of a chunk's queries over the paged cache.
//
// A long prompt is processed a chunk at a time ("How a serving engine actually
// works", paperfordummies.in, section "Prefill and decode are two different
// jobs"), and the block table grows by as many blocks as the chunk's tokens
// need ("Paged Attention and the Block Manager", snowch.github.io ch08, "The
// build").  A sequence whose cache holds L tokens after the step received its
// last n of them in the step (positions L-n .. L-1); the query of chunk token j
// (position L-n+j) attends to positions 0 .. L-n+j: the whole earlier context
// and the chunk up to itself.  With n = 1 this is a decode step.
//
// n-token append: new row x (of all sequences' packed rows) goes to the slot
// of its position, found through the block table; a wave per row.
//
// Attention: unlike decode, a chunk makes QK^T and PV real matrix products
// (n x G query rows against every key), so the work runs on the matrix cores.
// A query row is one (chunk token, head of the KV head's group) pair; rows of
// one (sequence, KV head) are ordered token-major.  A tile is 128 consecutive
// rows; a workgroup (one per compute unit, persistent) works through its
// share of the tiles one at a time, in two key groups of four waves, 32 rows
// per wave:
//   * the tiles are ranked longest first (by the position of their last row)
//     and dealt to the workgroups in rounds, alternating in direction, so
//     that every workgroup starts on a long tile and the short ones even out
//     the totals;
//   * each key group takes half of the tile's key iterations (64 keys each),
//     whose K and V tiles go from memory straight into LDS (two buffers for
//     K, two for V, 16-byte chunks XOR-swizzled by row);
//   * an iteration is two phases between workgroup barriers: M, all matrix
//     products (S^T = K Q^T of this iteration, O^T += V^T P^T of the one
//     before, v_mfma_f32_16x16x32), and V, all vector work (the prefix-causal
//     mask, the online softmax per row in base-2 units with a lazily moved
//     reference maximum, and the loads of later iterations); group 1 runs one
//     phase behind group 0 and each SIMD holds one wave of each, so one
//     wave's products overlap the other's softmax;
//   * the row sums come from the matrix core too, from the same rounded
//     weights as the outputs;
//   * at a tile's end the key groups' softmax states meet in LDS (the decode
//     merge's rule), each group writing half of the tile's output columns.
// Rows past L in a sequence's last block are loaded as zeros, so whatever
// those slots hold never reaches the output.
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_mfma.h"

namespace pkv {

// ---- n-token append ---------------------------------------------------------

// One wave per new row (its K and its V row), four rows per workgroup: the
// wave finds the row's sequence (a binary search of cu_new through the
// scalar cache; every lane agrees), then copies VB bytes per lane and pass.
constexpr int kAppendRowsPerBlock = 4;

template <int VB>
__global__ __launch_bounds__(kAppendRowsPerBlock * kWave) void append_tokens_kernel(AppendTokensParams p) {
    typedef const __attribute__((address_space(4))) int32_t cint;
    const cint* cu = (const cint*)p.cu_new;
    const int x = blockIdx.x * kAppendRowsPerBlock + wave_id_uniform();
    const int lane = threadIdx.x % kWave;
    const int S = p.num_seqs;
    if (x >= cu[S] || cu[0] > x) return;
    // the sequence owning row x: cu_new[s] <= x < cu_new[s + 1]
    int lo = 0, hi = S;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= x) lo = mid;
        else hi = mid;
    }
    const int s = lo;
    const int sp = ((const cint*)p.start_pos)[s];
    const int64_t pos = (int64_t)sp + (x - cu[s]);
    if (sp < 0 || pos < 0 || pos / p.block_size >= p.max_blocks) return;
    const int blk = ((const cint*)p.block_tables)[(int64_t)s * p.max_blocks + pos / p.block_size];
    if (blk < 0 || blk >= p.num_blocks) return;
    const int64_t slot = (int64_t)blk * p.block_size + pos % p.block_size;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        const char* src = static_cast<const char*>(kv ? p.v_new : p.k_new) + (int64_t)x * p.row_bytes;
        char* dst = static_cast<char*>(kv ? p.v_cache : p.k_cache) + slot * p.row_bytes;
        for (int off = lane * VB; off < p.row_bytes; off += kWave * VB) {
            if constexpr (VB == 16) {
                const v4u32_t v = *reinterpret_cast<const v4u32_t*>(src + off);
                *reinterpret_cast<v4u32_t*>(dst + off) = v;
            } else if constexpr (VB == 4) {
                *reinterpret_cast<uint32_t*>(dst + off) = *reinterpret_cast<const uint32_t*>(src + off);
            } else {
                *reinterpret_cast<uint16_t*>(dst + off) = *reinterpret_cast<const uint16_t*>(src + off);
            }
        }
    }
}

hipError_t launch_append_tokens(const AppendTokensParams& p, hipStream_t stream) {
    if (p.total <= 0 || p.num_seqs <= 0) return hipSuccess;
    const dim3 grid((p.total + kAppendRowsPerBlock - 1) / kAppendRowsPerBlock);
    const dim3 block(kAppendRowsPerBlock * kWave);
    if (p.row_bytes % 16 == 0)
        hipLaunchKernelGGL(append_tokens_kernel<16>, grid, block, 0, stream, p);
    else if (p.row_bytes % 4 == 0)
        hipLaunchKernelGGL(append_tokens_kernel<4>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(append_tokens_kernel<2>, grid, block, 0, stream, p);
    return hipGetLastError();
}

// ---- attention ---------------------------------------------------------------

// Shape of the attention workgroup: a tile of kPrefillRows query rows of one
// (sequence, KV head) in KS = 2 key groups of NW_ row waves; each wave owns
// NQ_ groups of 16 rows; an iteration covers NB = 4 blocks (64 keys).
template <int D, int NW_, int NQ_>
struct PrefillShape {
    static constexpr int NW = NW_;               // row waves per key group
    static constexpr int NQ = NQ_;               // 16-row groups per wave
    static constexpr int WAVES = 2 * NW;         // waves per workgroup
    static constexpr int PER_SIMD = WAVES / 4;   // waves per SIMD (one workgroup per CU)
    static constexpr int KS = 2;                 // key groups
    static constexpr int NB = 4;                 // 16-token tiles per iteration
    static constexpr int RB = D * 2;             // bytes per head row
    static constexpr int CH = RB / 16;           // 16-byte chunks per head row
    static constexpr int KK = D / 32;            // 16x16x32 products per score tile
    static constexpr int TT = D / 16;            // 16-wide output tiles
    static constexpr int ROWS_W = 16 * NQ;       // query rows per wave
    static constexpr int ROWS = NW * ROWS_W;     // query rows per tile
    static constexpr int TILE = kBlock * RB;     // bytes of one 16-token tile of one head
    static constexpr int SPAN = NB * TILE;       // an iteration's K (or V) rows of one group
    static constexpr int ARR = KS * SPAN;        // one LDS buffer: both groups' tiles
    static constexpr int RPR = 1024 / RB;        // rows per 1 KiB load instruction
    static constexpr int RG = kBlock / RPR;      // load instructions per 16-token tile
    static constexpr int PER_W = NB * RG / NW;   // load instructions per wave, iteration and cache
    static constexpr int STEP = NB * kBlock;     // keys per iteration
    static constexpr int TH = TT / 2;            // output tiles each key group writes
    static constexpr int HSTATE = TH * 4 + 2;    // floats a lane hands the other group (half of acc, m, l)
    static constexpr int HSQ = (HSTATE + 3) / 4; // of them in each of the four buffers
    static_assert(ROWS == kPrefillRows, "the grid's tile height");
    static_assert(CH == 4 * KK && D % 32 == 0, "head_dim a multiple of 32");
    static_assert(RPR * RB == 1024 && 8 % RPR == 0 && (NB * RG) % NW == 0,
                  "whole 1 KiB slices inside one block of 8 to 64, the same count per wave");
    static_assert(KS * NW * NQ * HSQ * kWave * 4 <= ARR, "both groups' handed-over state fits the four buffers");
};

// Word 3 of a raw buffer resource: 32-bit data format, no swizzle; with a
// stride of 0 the size (word 2) is in bytes and reads at or past it return 0.
constexpr int kBufferWord3 = 0x00020000;

// One wave's buffer load of 64 16-byte chunks straight into LDS: lane i reads
// `base + voff` (zeros at or past `bytes`) into `lds + 16 i`.  `base`, `bytes`
// and `lds` must be uniform over the wave.
__device__ __forceinline__ void lds_load_1k(const char* base, int bytes, char* lds, uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, __builtin_amdgcn_readfirstlane(bytes), kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// A block-table entry through the scalar cache (the index is uniform).
typedef const __attribute__((address_space(4))) int32_t prefill_const_i32;
__device__ __forceinline__ int scalar_entry(const int32_t* table, int i) {
    return ((prefill_const_i32*)table)[__builtin_amdgcn_readfirstlane(i)];
}

// The larger of two scores.  IEEE maximum (NaN-propagating) lowers to
// v_maximum3_f32 with no canonicalising max on inputs the compiler cannot
// prove canonical (lane exchange results, selects), which fmaxf needs; the
// scores are never NaN, so the two agree.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// The maximum over the four 16-lane rows' matching lanes (rows_max with smax).
__device__ __forceinline__ float rows_smax(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = smax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return smax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Headroom of the online softmax's reference maximum (log2 units): weights
// reach at most 2^8, well inside fp16 and bf16 range.
constexpr float kLazy = 8.f;

// Position of (row, 16-byte chunk) in an LDS tile of one head: rows of RB
// bytes, chunks XOR-swizzled by row so that transposed and row reads spread
// over the banks.
template <int RB>
__device__ __forceinline__ uint32_t tile_pos(int row, int chunk) {
    constexpr int CH = RB / 16;
    return (uint32_t)(row * RB + ((chunk ^ (row % CH)) * 16));
}

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with lgkmcnt(0), expcnt left open.
constexpr int waitcnt_vm_lgkm0(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }

// A workgroup barrier between phases.  No memory fence: a fence would also
// wait for every LDS load in flight, and the point of the phase barriers is
// to leave the next loads in flight (LDS reads finished before it, lgkmcnt
// 0, so no read can see a later write).  The empty asm statements keep memory
// accesses on their side of it and the scheduling barriers every other
// instruction: the phases only overlap the two key groups' work if each
// phase's products and softmax stay in it.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Ties a value to this point of the program: it must be computed before,
// and is taken as changed after, so the compiler can move its computation
// neither later (into the next phase) nor its uses earlier.
template <class T>
__device__ __forceinline__ void pin(T& x) {
    asm volatile("" : "+v"(x));
}

// ---- wave-wide integer reductions (every lane gets the result, uniform) ----
__device__ __forceinline__ int wave_sum_i32(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppQuadXor1, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppQuadXor2, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowHalfMirror, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowMirror, 0xF, 0xF, false);
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)a[0] + (int)a[1];
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return __builtin_amdgcn_readfirstlane((int)b[0] + (int)b[1]);
}

__device__ __forceinline__ int wave_max_i32(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, kDppQuadXor1, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, kDppQuadXor2, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, kDppRowHalfMirror, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, kDppRowMirror, 0xF, 0xF, false));
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = max((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return __builtin_amdgcn_readfirstlane(max((int)b[0], (int)b[1]));
}

// ---- tile order: longest first ----------------------------------------------
//
// Dealing tiles in decreasing key count approximates the longest-first list
// schedule: the long tiles start at once and the short ones fill in behind
// them, where the batch's order (sequence, tile) could leave a long tile for
// the end.  Tile t of a sequence covers
// chunk tokens [tQ, min((t+1)Q, n)) (Q = kPrefillRows / G) and reads keys 0 ..
// its last token's position.  The order sorts tiles by that last position,
// descending, ties by sequence; a sequence's tiles end at distinct positions,
// so each sequence has at most one tile per position.

// Tiles of a chunk of n tokens after ctx cached ones whose last position is
// at or past K.
template <int Q>
__device__ __forceinline__ int tiles_reaching(int ctx, int n, int K) {
    if (n <= 0 || ctx + n - 1 < K) return 0;
    const int nt = (n + Q - 1) / Q;
    // tile t < nt - 1 ends at ctx + (t + 1) Q - 1, which reaches K from t = (K - ctx) / Q on
    return nt - min(max(K - ctx, 0) / Q, nt - 1);
}

struct TileRef {
    int s, t;   // sequence (-1: no tile of this rank) and tile index within its chunk
    int q0;     // the sequence's first query row
    int L;      // its context length (clamped to its table)
    int n;      // its chunk length (the chunk's last n positions of L)
};

// The rank-th tile in that order, found by one wave alone: a search for the
// last position of that tile, counting the tiles that reach a position over
// all sequences, then its place among the tiles ending there, in sequence
// order.  Up to 64
// sequences the lanes test 64 positions per round; beyond, the lanes take
// sequences lane, lane + 64, ... and the search is four-way (three counts
// per round, their reductions interleaved).
template <int Q>
__device__ TileRef pick_tile(const PrefillParams& p, int rank, int lane, int max_len) {
    const int S = p.num_seqs;
    // Sequence s: first query row q0, context L, chunk nn; (ctx, n): tokens
    // before the chunk and chunk tokens computed (the first max_q_len); an
    // empty or impossible chunk has none.
    struct Seq {
        int q0, L, nn, ctx, n;
    };
    auto info = [&](int s) __attribute__((always_inline)) {
        Seq q;
        q.q0 = p.cu_q[s];
        q.L = min(max(p.context_lens[s], 0), max_len);
        q.nn = p.cu_q[s + 1] - q.q0;
        const bool ok = q.nn > 0 && q.nn <= q.L;
        q.ctx = ok ? q.L - q.nn : 0;
        q.n = ok ? min(q.nn, p.max_q_len) : 0;
        return q;
    };
    Seq q0{0, 0, 0, 0, 0};  // sequence `lane`
    if (lane < S) q0 = info(lane);
    auto count = [&](int K) __attribute__((always_inline)) {
        int c = tiles_reaching<Q>(q0.ctx, q0.n, K);
        for (int s = kWave + lane; s < S; s += kWave) {
            const Seq q = info(s);
            c += tiles_reaching<Q>(q.ctx, q.n, K);
        }
        return wave_sum_i32(c);
    };
    int last = q0.n > 0 ? q0.ctx + q0.n - 1 : -1;
    for (int s = kWave + lane; s < S; s += kWave) {
        const Seq q = info(s);
        if (q.n > 0) last = max(last, q.ctx + q.n - 1);
    }
    last = wave_max_i32(last);
    if (last < 0 || count(0) <= rank) return {-1, 0, 0, 0, 0};
    int lo = 0, hi = last + 1;  // count(lo) > rank >= count(hi) = 0
    int count_hi = 0;
    if (S <= kWave) {
        // Every lane holds one sequence, so each lane can count the tiles at
        // or past a threshold of its own over all of them (the sequences'
        // values broadcast by readlane): 64 thresholds per round, evenly
        // spread over (lo, hi); the ones whose count exceeds rank are a
        // prefix of the lanes.  Two rounds narrow 4096 positions to one.
        while (hi - lo > 1) {
            const int T = lo + 1 + (int)(((int64_t)lane * (hi - lo - 1)) >> 6);
            int c = 0;
            for (int s = 0; s < S; ++s)
                c += tiles_reaching<Q>(__builtin_amdgcn_readlane(q0.ctx, s), __builtin_amdgcn_readlane(q0.n, s), T);
            const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(c > rank));
            if (k > 0) lo = __builtin_amdgcn_readlane(T, k - 1);
            if (k < kWave) {
                hi = __builtin_amdgcn_readlane(T, k);
                count_hi = __builtin_amdgcn_readlane(c, k);
            }
        }
    }
    while (hi - lo >= 4) {
        const int d = hi - lo;
        const int m1 = lo + d / 4, m2 = lo + d / 2, m3 = lo + (3 * d) / 4;
        int c1 = tiles_reaching<Q>(q0.ctx, q0.n, m1), c2 = tiles_reaching<Q>(q0.ctx, q0.n, m2),
            c3 = tiles_reaching<Q>(q0.ctx, q0.n, m3);
        for (int s = kWave + lane; s < S; s += kWave) {
            const Seq q = info(s);
            c1 += tiles_reaching<Q>(q.ctx, q.n, m1);
            c2 += tiles_reaching<Q>(q.ctx, q.n, m2);
            c3 += tiles_reaching<Q>(q.ctx, q.n, m3);
        }
        c1 = wave_sum_i32(c1);
        c2 = wave_sum_i32(c2);
        c3 = wave_sum_i32(c3);
        if (c3 > rank) lo = m3;
        else if (c2 > rank) lo = m2, hi = m3, count_hi = c3;
        else if (c1 > rank) lo = m1, hi = m2, count_hi = c2;
        else hi = m1, count_hi = c1;
    }
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        const int cm = count(mid);
        if (cm > rank) lo = mid;
        else hi = mid, count_hi = cm;
    }
    int r = rank - count_hi;  // place among the tiles ending at lo (hi = lo + 1)
    for (int s0 = 0; s0 < S; s0 += kWave) {
        const int s = s0 + lane;
        Seq q = q0;
        if (s0 > 0) q = s < S ? info(s) : Seq{0, 0, 0, 0, 0};
        const bool has = s < S && tiles_reaching<Q>(q.ctx, q.n, lo) > tiles_reaching<Q>(q.ctx, q.n, lo + 1);
        uint64_t m = __builtin_amdgcn_ballot_w64(has);
        const int cnt = __builtin_popcountll(m);
        if (r < cnt) {
            for (int k = 0; k < r; ++k) m &= m - 1;
            const int sl = __builtin_ctzll(m);  // the lane holding it
            const int ctx = __builtin_amdgcn_readlane(q.ctx, sl), n = __builtin_amdgcn_readlane(q.n, sl);
            return {s0 + sl, (n + Q - 1) / Q - tiles_reaching<Q>(ctx, n, lo), __builtin_amdgcn_readlane(q.q0, sl),
                    __builtin_amdgcn_readlane(q.L, sl), __builtin_amdgcn_readlane(q.nn, sl)};
        }
        r -= cnt;
    }
    return {-1, 0, 0, 0, 0};
}

// The softmax weights as 16-bit matrix-core operands, four per lane and
// block, rounded to nearest even (fp16 keeps 11 significant bits, bf16 8).
// Row sums come from the same rounded weights (a product with a V^T of
// ones), so each output row is an exact convex combination of V rows under
// weights that differ from the true ones by a common factor and at most
// 2^-8 (bf16) each: the weights' rounding moves an output by at most 2^-8 of
// the spread of the V values its heavy keys hold, not of their size.
template <class E>
struct Weights;

template <>
struct Weights<F16> {
    typedef typename MfmaOps<F16>::op4_t op4_t;
    __device__ static __forceinline__ op4_t ones() { return op4_t{1.0f16, 1.0f16, 1.0f16, 1.0f16}; }
    __device__ static __forceinline__ op4_t pack(const float (&x)[4]) {
        return op4_t{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    }
};

template <>
struct Weights<BF16> {
    typedef typename MfmaOps<BF16>::op4_t op4_t;
    __device__ static __forceinline__ op4_t ones() { return op4_t{0x3F80, 0x3F80, 0x3F80, 0x3F80}; }
    __device__ static __forceinline__ op4_t pack(const float (&x)[4]) {
        return op4_t{__builtin_bit_cast(short, (__bf16)x[0]), __builtin_bit_cast(short, (__bf16)x[1]),
                     __builtin_bit_cast(short, (__bf16)x[2]), __builtin_bit_cast(short, (__bf16)x[3])};
    }
};

// Instruction classes of __builtin_amdgcn_sched_group_barrier (LLVM AMDGPU).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// One M phase's schedule (see the kernel): PV products steps of NQ products
// (plus the row sums' NQ at each block pair's end), each preceded by the
// fragment reads of the step AHEAD on, the last AHEAD steps by the scores'
// first reads instead (NQ KK q fragments and KK K fragments, spread over
// them); then NB scores blocks of NQ KK products, each preceded by the next
// block's KK K reads.
template <bool PV, bool QK, int U, int AHEAD, int TT, int NQ, int NB, int KK, int... I, int... B>
__device__ __forceinline__ void m_schedule(std::integer_sequence<int, I...>, std::integer_sequence<int, B...>) {
    constexpr int FIRST_QK = NQ * KK + KK;  // the scores' reads before their first products
    constexpr int TAIL = (FIRST_QK + AHEAD - 1) / AHEAD;
    if constexpr (PV) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * AHEAD, 0);
        auto step = [](auto u) __attribute__((always_inline)) {
            constexpr int i = decltype(u)::value;
            if constexpr (i + AHEAD < U) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            else if constexpr (QK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, TAIL, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, i % TT == TT - 1 ? 2 * NQ : NQ, 0);
        };
        (step(std::integral_constant<int, I>{}), ...);
    } else if constexpr (QK) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, FIRST_QK, 0);
    }
    if constexpr (QK) {
        auto block = [](auto b) __attribute__((always_inline)) {
            constexpr int i = decltype(b)::value;
            if constexpr (i + 1 < NB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, KK, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, NQ * KK, 0);
        };
        (block(std::integral_constant<int, B>{}), ...);
    }
}

// ---- the attention kernel -----------------------------------------------------
//
// Each key group takes half of the tile's key iterations (group 0 the first,
// group 1 the rest) and runs them as alternating phases, each ending at a
// workgroup barrier:
//   M_j: the output products of iteration j - 1 (O^T += V^T P^T, from V_{j-1}
//        in LDS) and the scores of iteration j (S^T = K Q^T, from K_j),
//   V_j: the loads of K_{j+2} and V_{j+1}, the causal mask and the softmax of
//        iteration j's scores (weights P_j, the lazy rescale of O and l),
// M_j all matrix-core work, V_j all vector work.  Group 1 runs one phase
// behind group 0, and each SIMD holds one wave of each group (waves w and
// w + 4 share a SIMD), so while one wave's products run on the matrix core
// the other wave's softmax runs on the vector ALU.  K and V have two LDS
// buffers each per group: K_j lives in K buffer j % 2 from V_{j-2} to M_j,
// V_j in V buffer j % 2 from V_{j-1} to M_{j+1}, so every load is issued
// three phases before its first reader; each wave waits (vmcnt) for its own
// loads at the end of the V phase before their reader.  B16: cache blocks of
// 16 tokens or more, so both halves of a wave's 16-token tile lie in one
// block and need one table entry and one placement.
template <class E, int D, int G, int NW, int NQ, bool B16>
__global__ __launch_bounds__(2 * NW * kWave, NW / 2) void prefill_kernel(PrefillParams p) {
    using SH = PrefillShape<D, NW, NQ>;
    static_assert(SH::WAVES == 2 * NW && SH::PER_SIMD == NW / 2, "the launch bounds above");
    using OPS = MfmaOps<E>;
    using op4_t = typename OPS::op4_t;
    constexpr int RB = SH::RB, CH = SH::CH, KK = SH::KK, TT = SH::TT, NB = SH::NB;
    constexpr int PER_W = SH::PER_W, STEP = SH::STEP;
    constexpr int PV_STEPS = (NB / 2) * TT;  // products steps (block pair, output tile) per iteration
    constexpr int PV_AHEAD = 4;              // steps whose V fragments are in flight
    constexpr int Q = kPrefillRows / G;  // chunk tokens per tile
    // Four separate arrays, so the compiler can tell the loads filling one
    // buffer from the reads of another and waits only where they meet.
    __shared__ __attribute__((aligned(16))) char lds_k0[SH::ARR];
    __shared__ __attribute__((aligned(16))) char lds_k1[SH::ARR];
    __shared__ __attribute__((aligned(16))) char lds_v0[SH::ARR];
    __shared__ __attribute__((aligned(16))) char lds_v1[SH::ARR];
    // The tile's q rows (both key groups use the same), XOR-swizzled like K:
    // read back for each iteration's scores rather than held in registers,
    // which leaves room to read the V and K fragments well ahead.
    __shared__ __attribute__((aligned(16))) char lds_q[SH::ROWS * RB];

    // A persistent grid: W workgroups per KV head, KV head fastest, so the
    // XCDs (which take workgroups round-robin) each get the same mix, and a
    // head's tiles all run on one XCD (its K and V stay in that XCD's L2)
    // when Hkv is a multiple of 8.  Slot j of a head takes the tiles of ranks
    // j, 2W - 1 - j, 2W + j, 4W - 1 - j, ... in the longest-first order: the
    // first round deals the W longest tiles one each, the second gives the
    // shortest of the next W to the slot that got the longest, and so on.
    const int Hkv = p.n_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int W = gridDim.x / Hkv;
    const int sj = blockIdx.x / Hkv;
    const int R = p.num_seqs * ((p.max_q_len * G + SH::ROWS - 1) / SH::ROWS);  // ranks, at most
    const int lane = threadIdx.x % kWave;
    const int max_len = p.max_blocks << p.block_shift;
    // The slot's tiles are found SH::WAVES at a time, one per wave, and handed
    // over through LDS (the start of the last V buffer, whose first load
    // comes phases later); lane k of `ref` holds the round's k-th tile as
    // sequence << 16 | tile, unsigned (all ones: none; a tile index stays
    // below kMaxPrefillTiles = 65535), and lane k of ref_q0, ref_n and ref_L
    // its sequence's first query row, chunk length and (clamped) context
    // length, so a tile starts without another memory round trip.
    static_assert(kMaxPrefillTiles <= 65535, "the tile index fits 16 bits, below 0xffff");
    int ref = -1, ref_q0 = 0, ref_n = 0, ref_L = 0;
    for (int item = 0;; ++item) {
        // the last tile's state reads (all four K/V buffers) are done before
        // this tile's loads go into them; its output stores need not be (a
        // __syncthreads would also wait for those)
        if (item > 0) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
            phase_barrier();
        }
        const int k_round = item % SH::WAVES;
        if (k_round == 0) {
            int* sh = reinterpret_cast<int*>(lds_v1);
            const int wv = wave_id_uniform();
            const int it = item + wv;
            const int rank = it * W + ((it & 1) ? W - 1 - sj : sj);
            // (an opaque lane index: hoisted out of the loop, the search's
            // per-lane addresses would hold registers through every tile)
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const TileRef t = rank < R ? pick_tile<Q>(p, rank, ln, max_len) : TileRef{-1, 0, 0, 0, 0};
            if (lane == 0) {
                sh[wv] = t.s < 0 ? -1 : (int)((uint32_t)t.s << 16 | (uint32_t)t.t);
                sh[SH::WAVES + wv] = t.q0;
                sh[2 * SH::WAVES + wv] = t.n;
                sh[3 * SH::WAVES + wv] = t.L;
            }
            __syncthreads();
            const bool in = lane < SH::WAVES;
            ref = in ? sh[lane] : -1;
            ref_q0 = in ? sh[SH::WAVES + lane] : 0;
            ref_n = in ? sh[2 * SH::WAVES + lane] : 0;
            ref_L = in ? sh[3 * SH::WAVES + lane] : 0;
        }
        const int cur = __builtin_amdgcn_readlane(ref, k_round);
        if (cur == -1) break;  // ranks past the batch's tiles: so are the slot's later ones
        TileRef tr;
        tr.s = (int)((uint32_t)cur >> 16);
        tr.t = cur & 0xffff;
        tr.q0 = __builtin_amdgcn_readlane(ref_q0, k_round);
        tr.n = __builtin_amdgcn_readlane(ref_n, k_round);
        tr.L = __builtin_amdgcn_readlane(ref_L, k_round);
        const int s = tr.s;
        const int q0 = tr.q0;
        const int n = tr.n;
        const int L = tr.L;
        const int Hq = p.n_q_heads;
        const int nrows = min(n, p.max_q_len) * G;  // rows computed
        const int r0 = tr.t * SH::ROWS;
        const int ctx = L - n;  // tokens before the chunk
        const int wg_last_pos = ctx + (min(r0 + SH::ROWS, nrows) - 1) / G;
        const int nblk = wg_last_pos / kBlock + 1;  // 16-token tiles the workgroup reads
        const int nit = (nblk + NB - 1) / NB;
        const int NJ = (nit + 1) / 2;                // phase pairs of either group

        const int kg = wave_id_uniform() / SH::NW;  // key group
        const int w = wave_id_uniform() % SH::NW;   // row wave within the group
        const int kb = kg == 0 ? 0 : NJ;            // the group's first iteration
        const int nj = kg == 0 ? NJ : nit - NJ;     // and its count
        const int gq = lane / 16;  // MFMA lane coordinates
        const int jq = lane % 16;
        const int wr0 = r0 + w * SH::ROWS_W;  // this wave's first row
        const int wave_first_pos = ctx + wr0 / G;
        // Iteration j of the group is masked unless every key of it is visible to
        // every row of the wave.  A wave computes every phase of its group, also
        // for an iteration none of its rows sees (or one past the group's range,
        // loaded as zeros): the mask makes all its weights 0, and skipping it
        // would not shorten the phase, which waits for every wave at its barrier.
        auto masked = [&](int j) __attribute__((always_inline)) { return (kb + j + 1) * STEP - 1 > wave_first_pos; };

        // The softmax below needs a positive scale: a negative one moves into q's
        // sign bits (exact), and a zero one becomes the smallest normal float,
        // which leaves every weight at exactly 1 as zero would (|score| x 2^-126
        // is far below half an ulp of 1 for any 16-bit q and K).
        const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
        const float scale_log2 = fmaxf(fabsf(p.scale_log2), 1.17549435e-38f);
        // q rows of this wave: group c, column jq is row wr0 + 16c + jq (row
        // 32w + 16c + jq of the tile); group 0's waves load them here and put
        // them in LDS in the prologue (rows past the chunk as zeros), once the
        // first K and V loads are under way; the first barrier publishes them.
        int qpos[NQ];
        Vec16 qv[NQ][KK];
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int row = wr0 + 16 * c + jq;
            const bool ok = row < nrows;
            const int tok = row / G;
            qpos[c] = ok ? ctx + tok : -1;
            const char* qrow = static_cast<const char*>(p.q) + (((int64_t)(q0 + tok) * Hq + kvh * G + row % G) * D) * 2;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                qv[c][kk] = ok && kg == 0 ? load16(qrow + (4 * kk + gq) * 16) : Vec16{{0u, 0u, 0u, 0u}};
        }
        // Row state: reference maximum m, output acc and the weights' sum, which
        // the matrix core accumulates too (the product with a V^T of ones puts
        // row jq's sum in every element of lane column jq).
        float m[NQ];
        f32x4_t acc[NQ][TT], lsum[NQ];
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            m[c] = -INFINITY;
            lsum[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[c][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const op4_t ones = Weights<E>::ones();

        // K and V go from memory straight into LDS (buffer loads with an LDS
        // destination).  One such instruction of a wave fills a contiguous 1 KiB
        // of LDS, lane i bytes 16i .. 16i+15: RPR rows of one 16-token tile of one
        // cache, which lie in one cache block whatever the block size (RPR divides
        // 8).  Lane i fetches the global chunk that the row's XOR swizzle puts in
        // its slot.  The block's base address and the bytes of its rows inside the
        // sequence make the buffer resource, so rows past the context and invalid
        // table entries arrive as zeros (out-of-range buffer reads return 0).
        // Slice g = w + k NW of an iteration (per cache): tile g / RG, rows
        // RPR (g % RG) ..; an iteration spans a whole number of blocks, so the
        // slice's row offset inside its block is the same in every iteration and
        // goes into the lane offsets.
        // Wave w of a key group loads tile w of each iteration (K and V): slice
        // k is rows RPR k .. RPR k + RPR - 1 of it, inside the tile's first eight
        // rows (half 0) or its last eight (half 1); with blocks of 16 tokens or
        // more the two halves are one block.
        static_assert(SH::NW == NB && SH::PER_W == SH::RG, "one 16-token tile per row wave");
        const uint32_t row_stride = (uint32_t)Hkv * RB;
        const int bshift = p.block_shift;
        const int bsize = 1 << bshift;
        const uint32_t blk_bytes = row_stride << bshift;  // below 2^32: 64 x Hkv x 256 bytes at most
        const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * RB;
        const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * RB;
        const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks;
        const int tt0 = kb * STEP + w * kBlock;  // first token of the wave's tile in the group's iteration 0
        uint32_t voff[PER_W];
#pragma unroll
        for (int k = 0; k < PER_W; ++k) {
            const int row = k * SH::RPR + lane / CH;  // row in the tile
            voff[k] = (uint32_t)(((tt0 + k * SH::RPR) & (bsize - 1)) + lane / CH) * row_stride +
                      (uint32_t)(((lane % CH) ^ (row % CH)) * 16);
        }
        // halves past the workgroup's last tile, or past the sequence's last table entry, load nothing
        const int tok_lim = min(nblk * kBlock, (L + bsize - 1) & -bsize);
        typedef int Ents[2];
        struct Blk {
            uint64_t off;  // byte offset of the half's block in a cache
            int size;      // bytes of its rows inside the sequence (0: load zeros)
        };
        // Table entries of the two halves of the group's iteration j, read a
        // phase before their loads.  The read index is clamped into the table and
        // nothing depends on the value until then, so no read waits or branches.
        auto entries = [&](int j, Ents& e) __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < (B16 ? 1 : 2); ++h)
                e[h] = scalar_entry(table, min(j * STEP + tt0 + 8 * h, tok_lim - 1) >> bshift);
            if constexpr (B16) e[1] = e[0];
        };
        // Where the halves of iteration j come from; a half past the workgroup's
        // keys, or of an iteration past the group's range, loads zeros (its loads
        // still run, so that every phase issues the same number of loads and the
        // waits are static).
        auto place = [&](int j, const Ents& e, Blk (&bl)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < (B16 ? 1 : 2); ++h) {
                const int tok = j * STEP + tt0 + 8 * h;
                const bool ok = j < nj && tok < tok_lim && (uint32_t)e[h] < (uint32_t)p.num_blocks;
                bl[h].off = (uint64_t)(uint32_t)(ok ? e[h] : 0) * blk_bytes;
                bl[h].size = ok ? min(L - (tok & -bsize), bsize) * (int)row_stride : 0;
            }
            // (the second half's token is 8 past the first, in the same block, and
            // tok_lim is a multiple of 16, so its placement is the first's)
            if constexpr (B16) bl[1] = bl[0];
        };
        // (The slice's LDS offset is formed at each use from one opaque value:
        // left to itself the compiler would keep an offset per buffer and slice
        // in scalar registers, which it has too few of here.)
        const uint32_t wslot = (uint32_t)(kg * SH::SPAN + w * SH::TILE);
        auto issue = [&](char* buf, const char* base, const Blk (&bl)[2]) __attribute__((always_inline)) {
            uint32_t ws = wslot;
            asm volatile("" : "+s"(ws));
#pragma unroll
            for (int k = 0; k < PER_W; ++k) {
                const Blk& b = bl[(k * SH::RPR) / 8];
                lds_load_1k(base + b.off, b.size, buf + ws + k * 1024, voff[k]);
            }
        };

        f32x4_t sc[NQ][NB];            // scores of an iteration, from its M phase to its V phase
        op4_t ph[NQ][NB];              // its weights, from its V phase to the next M
        // S^T = K Q^T of iteration j: lane (gq, jq) holds keys 16 nb + 4 gq + r of
        // row column jq.  Every block gets its products, those past the wave's
        // rows included (the softmax masks them): a branch around them would put
        // the first reads of a product's result right after it, closer than its
        // latency.
        auto scores = [&](const char* kl) __attribute__((always_inline)) {
            Vec16 qf[NQ][KK];
#pragma unroll
            for (int c = 0; c < NQ; ++c)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    qf[c][kk] = lds_load16(lds_q, tile_pos<RB>(w * SH::ROWS_W + 16 * c + jq, 4 * kk + gq));
            // block nb's K fragments are read a block before its products
            constexpr int AHEAD = 1;
            Vec16 ka[NB][KK];
            auto fetch = [&](int nb) __attribute__((always_inline)) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[nb][kk] = lds_load16(kl + nb * SH::TILE, tile_pos<RB>(jq, 4 * kk + gq));
            };
#pragma unroll
            for (int nb = 0; nb < AHEAD; ++nb) fetch(nb);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (nb + AHEAD < NB) fetch(nb + AHEAD);
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    sc[c][nb] = OPS::qk(ka[nb][0], qf[c][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int kk = 1; kk < KK; ++kk) sc[c][nb] = OPS::qk(ka[nb][kk], qf[c][kk], sc[c][nb]);
                }
            }
        };
        // Online softmax of the scores: weights in base-2 units against a lazily
        // moved reference maximum m (it moves only when a row's scores pass it by
        // more than kLazy, so weights stay below 2^kLazy and most iterations skip
        // the rescale of O and l).
        auto softmax = [&](int j) __attribute__((always_inline)) {
            // The prefix-causal mask: a key past the row's position scores -inf
            // (every key of an unmasked iteration is visible to every row).  A
            // bitwise select on the sign of lim - key, which the compiler turns
            // into a compare and a select through VCC one element at a time
            // (compares hoisted ahead of their selects would each hold a scalar
            // register pair).
            if (masked(j)) {
                const int key0 = (kb + j) * STEP;
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const int lim = qpos[c] - key0 - 4 * gq;  // last visible key offset of this lane
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const uint32_t msk = (uint32_t)((lim - (16 * nb + r)) >> 31);
                            sc[c][nb][r] =
                                __uint_as_float((msk & 0xff800000u) | (~msk & __float_as_uint(sc[c][nb][r])));
                        }
                }
            }
            // each lane's largest score of each row group, as a tree
            float mx[NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                float t4[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    t4[nb] = smax(smax(sc[c][nb][0], sc[c][nb][1]), smax(sc[c][nb][2], sc[c][nb][3]));
                mx[c] = smax(smax(t4[0], t4[1]), smax(t4[2], t4[3]));
                static_assert(NB == 4, "the tree above");
            }
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                // The reference moves when some row's largest scaled score passes
                // it by more than kLazy, i.e. when some lane's does: the row's
                // maximum over its four lanes is needed only then.
                if (__builtin_amdgcn_ballot_w64(mx[c] * scale_log2 > m[c] + kLazy)) {
                    const float mn = rows_smax(mx[c]) * scale_log2;  // the row's largest scaled score here
                    const float nm = fmaxf(m[c], mn);
                    const float alpha = __builtin_amdgcn_exp2f(m[c] - (nm == -INFINITY ? 0.f : nm));
                    lsum[c] *= alpha;
#pragma unroll
                    for (int t = 0; t < TT; ++t) acc[c][t] *= alpha;
                    m[c] = nm;
                }
                const float ms = m[c] == -INFINITY ? 0.f : m[c];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float pr[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(sc[c][nb][r], scale_log2, -ms));
                    ph[c][nb] = Weights<E>::pack(pr);
                    pin(ph[c][nb]);
                }
            }
        };
        // O^T += V^T P^T of iteration j.  V^T is read transposed: lane (gq, jq)
        // takes key row 4gq + jq/4, bytes 32t + 8(jq%4).  Blocks nb and nb + 1 make
        // one 16x16x32 product: contraction slots 0-3 are keys 4gq + r of block
        // nb, slots 4-7 those of block nb + 1, in V^T and P^T alike.  The
        // fragments of step u (pair u / TT, output tile u % TT) are read AHEAD
        // steps ahead of their products, so that the reads' latency hides behind
        // them.  Also the weights' row sums (a V^T of ones).
        auto products = [&](const char* vl) __attribute__((always_inline)) {
            constexpr int U = PV_STEPS, AHEAD = PV_AHEAD;
            const int trow = 4 * gq + jq / 4;
            op4_t fa[U], fb[U];
            auto fetch = [&](int u) __attribute__((always_inline)) {
                const int nb = 2 * (u / TT), t = u % TT;
                const uint32_t off = tile_pos<RB>(trow, 2 * t + (jq % 4) / 2) + 8 * (jq % 2);
                fa[u] = OPS::read_tr(vl + nb * SH::TILE + off);
                fb[u] = OPS::read_tr(vl + (nb + 1) * SH::TILE + off);
            };
#pragma unroll
            for (int u = 0; u < AHEAD; ++u) fetch(u);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u + AHEAD < U) fetch(u + AHEAD);
                const int nb = 2 * (u / TT), t = u % TT;
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    acc[c][t] = OPS::pv2(fa[u], fb[u], ph[c][nb], ph[c][nb + 1], acc[c][t]);
                }
                if (t == TT - 1) {
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        lsum[c] = OPS::pv2(ones, ones, ph[c][nb], ph[c][nb + 1], lsum[c]);
                    }
                }
            }
        };

        // Phase M_j (buffer parity b = j % 2): the products of j - 1 from V
        // buffer 1 - b (their weights die there), then the scores of j from K
        // buffer b (born there), so weights and scores never hold registers
        // together.
        Ents ec;     // table entries of iteration j + 2 when V_j starts
        Blk bl[2];   // where iteration j + 1's halves come from when V_j starts
        // (M_0 has no products, the last M phase, M_NJ, no scores)
        auto mphase = [&](int j, auto par, auto pv, auto qk) __attribute__((always_inline)) {
            constexpr int b = decltype(par)::value;
            // The products are the phase's critical path: this wave issues first
            // (the SIMD otherwise favours the older wave, group 0's), and its
            // partner's softmax fills the cycles between the products.
            __builtin_amdgcn_s_setprio(1);
            if constexpr (decltype(pv)::value) products((b ? lds_v0 : lds_v1) + kg * SH::SPAN);
            if constexpr (decltype(qk)::value) {
                scores((b ? lds_k1 : lds_k0) + kg * SH::SPAN);
#pragma unroll
                for (int c = 0; c < NQ; ++c)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) pin(sc[c][nb]);
            }
            // The phase's order through scheduling: the products' first fragment
            // reads, then per products step the reads PV_AHEAD steps on (in the
            // last steps, the scores' q and first K reads) and the step's
            // products; then per scores block the next block's K reads and the
            // block's products.
            m_schedule<decltype(pv)::value, decltype(qk)::value, PV_STEPS, PV_AHEAD, TT, NQ, NB, KK>(
                std::make_integer_sequence<int, PV_STEPS>{}, std::make_integer_sequence<int, NB>{});
            __builtin_amdgcn_s_setprio(0);
        };
        // Phase V_j: the loads of K_{j+2} into K buffer b (last read by the
        // group's scores in M_j) and of V_{j+1} into V buffer 1 - b (last read by
        // the products in M_j), the table entries of j + 3, the softmax of j;
        // then this wave's loads of K_{j+1} and V_j, issued in V_{j-1}, land
        // (this phase's stay in flight), so that after the barrier the whole
        // group's K_{j+1} and V_j are in LDS.
        auto vphase = [&](int j, auto par) __attribute__((always_inline)) {
            constexpr int b = decltype(par)::value;
            Blk b2[2];
            place(j + 2, ec, b2);
            issue(b ? lds_k1 : lds_k0, kbase, b2);
            issue(b ? lds_v0 : lds_v1, vbase, bl);
#pragma unroll
            for (int h = 0; h < 2; ++h) bl[h] = b2[h];
            entries(j + 3, ec);
            softmax(j);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * PER_W));
        };

        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        // Prologue: the loads of K_0, V_0 and K_1, then q into LDS; K_0 (and q)
        // land before the first barrier.
        {
            Ents e1;
            entries(0, ec);
            entries(1, e1);
            place(0, ec, bl);
            issue(lds_k0, kbase, bl);
            issue(lds_v0, vbase, bl);
            place(1, e1, bl);
            issue(lds_k1, kbase, bl);
            entries(2, ec);
            if (kg == 0) {
#pragma unroll
                for (int c = 0; c < NQ; ++c)
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) {
                        Vec16 v = qv[c][kk];
#pragma unroll
                        for (int e = 0; e < 4; ++e) v.w[e] ^= qsign;
                        lds_store16(lds_q, tile_pos<RB>(w * SH::ROWS_W + 16 * c + jq, 4 * kk + gq), v);
                    }
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * PER_W));
        }
        phase_barrier();
        if (kg == 1) phase_barrier();  // group 1 runs one phase behind
        using T = std::true_type;
        using F = std::false_type;
        mphase(0, B0{}, F{}, T{});
        phase_barrier();
        vphase(0, B0{});
        phase_barrier();
        int j = 1;
        for (; j + 1 < NJ; j += 2) {
            mphase(j, B1{}, T{}, T{});
            phase_barrier();
            vphase(j, B1{});
            phase_barrier();
            mphase(j + 1, B0{}, T{}, T{});
            phase_barrier();
            vphase(j + 1, B0{});
            phase_barrier();
        }
        if (j < NJ) {  // j odd
            mphase(j, B1{}, T{}, T{});
            phase_barrier();
            vphase(j, B1{});
            phase_barrier();
        }
        // M_NJ: the last products; then the last phases' zero fills land before
        // the buffers take group 1's state.
        if (NJ & 1) mphase(NJ, B1{}, T{}, F{});
        else mphase(NJ, B0{}, T{}, F{});
        __builtin_amdgcn_s_waitcnt(0);
        phase_barrier();
        if (kg == 0) phase_barrier();

        float l[NQ];
#pragma unroll
        for (int c = 0; c < NQ; ++c) l[c] = lsum[c][0];
        // The key groups' states meet in LDS (every load has landed and every read
        // finished before the last barriers): each group hands the other the half
        // of its accumulator that the other writes out (group 0 writes output
        // tiles 0 .. TH - 1, group 1 the rest) with its m and l, and both fold the
        // two states with the decode merge's rule, the same arithmetic in either
        // group.  Element e of group g's handed-over state for row group c goes to
        // buffer e % 4, lane-major, so each store and load is one conflict-free
        // row of 64 words.
        constexpr int TH = SH::TH;
        auto slot = [&](int g, int c, int e) __attribute__((always_inline)) -> float* {
            char* arr = e % 4 == 0 ? lds_k0 : e % 4 == 1 ? lds_k1 : e % 4 == 2 ? lds_v0 : lds_v1;
            return reinterpret_cast<float*>(arr) + ((((g * SH::NW + w) * NQ + c) * SH::HSQ + e / 4) * kWave + lane);
        };
        auto hand_over = [&](auto kgc) __attribute__((always_inline)) {
            constexpr int KG = decltype(kgc)::value;
            constexpr int GIVE = KG == 0 ? TH : 0;  // first output tile handed over
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
#pragma unroll
                for (int h = 0; h < TH; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) *slot(KG, c, 4 * h + r) = acc[c][GIVE + h][r];
                *slot(KG, c, 4 * TH) = m[c];
                *slot(KG, c, 4 * TH + 1) = l[c];
            }
        };
        auto fold = [&](auto kgc) __attribute__((always_inline)) {
            constexpr int KG = decltype(kgc)::value;
            constexpr int KEEP = KG == 0 ? 0 : TH;  // first output tile written here
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                // group 0's and group 1's m and l
                const float mo = *slot(1 - KG, c, 4 * TH), lo = *slot(1 - KG, c, 4 * TH + 1);
                const float m0 = KG == 0 ? m[c] : mo, m1 = KG == 0 ? mo : m[c];
                const float l0 = KG == 0 ? l[c] : lo, l1 = KG == 0 ? lo : l[c];
                const float mm = fmaxf(m0, m1);
                const float mr = mm == -INFINITY ? 0.f : mm;
                const float a0 = __builtin_amdgcn_exp2f(m0 - mr);
                const float a1 = __builtin_amdgcn_exp2f(m1 - mr);
                const float lt = fmaf(l1, a1, l0 * a0);
                const int row = wr0 + 16 * c + jq;
                if (row >= nrows) continue;
                const float inv = 1.f / lt;
                char* orow = static_cast<char*>(p.out) + (((int64_t)(q0 + row / G) * Hq + kvh * G + row % G) * D) * 2;
#pragma unroll
                for (int h = 0; h < TH; ++h) {
                    float o[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float own = acc[c][KEEP + h][r], oth = *slot(1 - KG, c, 4 * h + r);
                        o[r] = fmaf(KG == 0 ? oth : own, a1, (KG == 0 ? own : oth) * a0) * inv;
                    }
                    store4<E>(orow + (16 * (KEEP + h) + 4 * gq) * 2, o[0], o[1], o[2], o[3]);
                }
            }
        };
        using K0 = std::integral_constant<int, 0>;
        using K1 = std::integral_constant<int, 1>;
        if (kg == 0) hand_over(K0{});
        else hand_over(K1{});
        __syncthreads();
        if (kg == 0) fold(K0{});
        else fold(K1{});
    }  // the slot's next tile
}

// Launch shape: 8 waves (two key groups of four) over 128-row tiles, 32 rows
// per wave, 4 blocks (64 keys) per iteration: 32 KiB (head_dim 128) or 16 KiB
// (64) per K or V buffer, four buffers and the tile's q, two waves per SIMD.
template <class E, int D, int G, int NW = 4, int NQ = 2>
static hipError_t launch_prefill_g(const PrefillParams& p, hipStream_t stream) {
    using SH = PrefillShape<D, NW, NQ>;
    const int64_t tiles = ((int64_t)p.max_q_len * G + SH::ROWS - 1) / SH::ROWS;
    if (tiles > kMaxPrefillTiles || p.num_seqs > 65535 || tiles * p.num_seqs > INT32_MAX)
        return hipErrorInvalidConfiguration;
    // W workgroups per KV head, one per compute unit (a workgroup takes the
    // whole LDS), at most one per rank.
    static thread_local int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev != cached_dev) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cached_dev = dev;
        cached_cus = cus;
    }
    const int64_t ranks = tiles * p.num_seqs;
    const int64_t W = std::max<int64_t>(1, std::min<int64_t>(ranks, cached_cus / p.n_kv_heads));
    auto kern = p.block_shift >= 4 ? prefill_kernel<E, D, G, NW, NQ, true> : prefill_kernel<E, D, G, NW, NQ, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(W * p.n_kv_heads)), dim3(SH::WAVES * kWave), 0, stream, p);
    return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_prefill_d(const PrefillParams& p, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_prefill_g<E, D, 1>(p, stream);
        case 2: return launch_prefill_g<E, D, 2>(p, stream);
        case 4: return launch_prefill_g<E, D, 4>(p, stream);
        case 8: return launch_prefill_g<E, D, 8>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
static hipError_t launch_prefill_e(const PrefillParams& p, int head_dim, int group, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_prefill_d<E, 64>(p, group, stream);
        case 128: return launch_prefill_d<E, 128>(p, group, stream);
        default: return hipErrorInvalidValue;
    }
}

bool prefill_supported(int dtype, int head_dim, int group) {
    return (dtype == 1 || dtype == 2) && (head_dim == 64 || head_dim == 128) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int group, hipStream_t stream) {
    if (p.num_seqs <= 0 || p.max_q_len <= 0) return hipSuccess;
    switch (dtype) {
        case 1: return launch_prefill_e<F16>(p, head_dim, group, stream);
        case 2: return launch_prefill_e<BF16>(p, head_dim, group, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
