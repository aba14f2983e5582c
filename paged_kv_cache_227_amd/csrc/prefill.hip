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
// n-token append: workgroup x copies new row x (of all sequences' packed rows)
// into the slot of its position, found through the block table.
//
// Attention: unlike decode, a chunk makes QK^T and PV real matrix products
// (n x G query rows against every key), so the work runs on the matrix cores.
// A query row is one (chunk token, head of the KV head's group) pair; rows of
// one (sequence, KV head) are ordered token-major.  A workgroup holds one tile
// of NW x 16 x NQ consecutive rows, in KS key groups of NW waves:
//   * each key group takes its share of the tile's key iterations; an
//     iteration's K and V tiles (NB blocks) are loaded once per group (the
//     table entries first, then every 16-byte load in flight at once, one
//     iteration ahead of the compute) and stored in LDS, double-buffered,
//     16-byte chunks XOR-swizzled by row;
//   * each wave owns NQ groups of 16 rows.  Per block and group:
//       S^T = K Q^T   (v_mfma_f32_16x16x32, K from LDS as the A operand, the
//                      group's q rows as B, held in registers),
//     the prefix-causal mask (key position <= the row's position) entering as
//     the products' initial value (0 or -inf) in the steps that need it, an
//     online softmax per row in base-2 units with a lazily moved reference
//     maximum (each row's state lives in one lane column), then, for each
//     pair of blocks,
//       O^T += V^T P^T (v_mfma_f32_16x16x32, V^T read transposed from LDS,
//                      P^T straight from S^T's accumulator layout; the two
//                      blocks' 4-key lane slices make the 8 contraction slots),
//     with P split into high and low 16-bit parts for bf16 so about 16 bits of
//     each weight survive;
//   * the key groups' softmax states meet in LDS at the end (the decode merge's
//     rule), and group 0 writes the rows;
//   * iterations wholly past a wave's last position are skipped by that wave.
// Rows past L in a sequence's last block are loaded as zeros, so whatever
// those slots hold never reaches the output.
#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_mfma.h"

namespace pkv {

// ---- n-token append ---------------------------------------------------------

template <int VB>
__global__ __launch_bounds__(256) void append_tokens_kernel(AppendTokensParams p) {
    const int x = blockIdx.x;
    const int S = p.num_seqs;
    if (x >= p.cu_new[S] || p.cu_new[0] > x) return;
    // the sequence owning row x: cu_new[s] <= x < cu_new[s + 1]
    int lo = 0, hi = S;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_new[mid] <= x) lo = mid;
        else hi = mid;
    }
    const int s = lo;
    const int64_t pos = (int64_t)p.start_pos[s] + (x - p.cu_new[s]);
    if (p.start_pos[s] < 0 || pos < 0 || pos / p.block_size >= p.max_blocks) return;
    const int blk = p.block_tables[(int64_t)s * p.max_blocks + pos / p.block_size];
    if (blk < 0 || blk >= p.num_blocks) return;
    const int64_t slot = (int64_t)blk * p.block_size + pos % p.block_size;
    const bool is_v = blockIdx.y != 0;
    const char* src = static_cast<const char*>(is_v ? p.v_new : p.k_new) + (int64_t)x * p.row_bytes;
    char* dst = static_cast<char*>(is_v ? p.v_cache : p.k_cache) + slot * p.row_bytes;
    for (int off = threadIdx.x * VB; off < p.row_bytes; off += blockDim.x * VB) {
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

hipError_t launch_append_tokens(const AppendTokensParams& p, hipStream_t stream) {
    if (p.total <= 0 || p.num_seqs <= 0) return hipSuccess;
    const dim3 grid(p.total, 2);
    if (p.row_bytes % 16 == 0)
        hipLaunchKernelGGL(append_tokens_kernel<16>, grid, dim3(256), 0, stream, p);
    else if (p.row_bytes % 4 == 0)
        hipLaunchKernelGGL(append_tokens_kernel<4>, grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(append_tokens_kernel<2>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ---- attention ---------------------------------------------------------------

template <class E, int D, int G, int NW, int NQ, int NB, int KS>
struct PrefillShape {
    static constexpr int RB = D * 2;            // bytes per head row
    static constexpr int CH = RB / 16;          // 16-byte chunks per head row
    static constexpr int KK = D / 32;           // 16x16x32 products per score tile
    static constexpr int TT = D / 16;           // 16-wide output tiles
    static constexpr int ROWS_W = 16 * NQ;      // query rows per wave
    static constexpr int ROWS = NW * ROWS_W;    // query rows per workgroup
    static constexpr int TILE = kBlock * RB;    // bytes of one block's K (or V) rows of one head
    static constexpr int SPAN = NB * TILE;      // bytes of an iteration's K (or V) rows
    static constexpr int BUF_BYTES = KS * 2 * SPAN;      // one buffer: [group][K, V] tiles
    static constexpr int STATE = TT * 4 + 2;             // floats of one lane's row state (acc, m, l)
    // Group 1's states go to the two (by then idle) buffers, half each, when
    // they fit there, else to an array of their own.
    static constexpr int STATE_A = (STATE + 1) / 2;      // floats in the first buffer
    static constexpr bool STATE_IN_BUFFERS = KS > 1 && NW * NQ * STATE_A * kWave * 4 <= BUF_BYTES;
    static constexpr int MERGE_BYTES = KS > 1 && !STATE_IN_BUFFERS ? NW * NQ * STATE * kWave * 4 : 16;
    static_assert(E::kBytes == 2 && D % 32 == 0 && CH == 4 * KK, "16-bit caches, head_dim a multiple of 32");
    static_assert(NB % 2 == 0, "PV takes blocks in pairs");
    static_assert(KS == 1 || KS == 2, "one or two key groups");
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

// One iteration covers NB consecutive blocks: their K and V tiles are loaded
// together (one iteration ahead) and one softmax rescale covers all NB x 16 keys.
// With KS = 2 the workgroup holds two key groups of NW waves over the same rows:
// group 0 takes the first half of the iterations, group 1 the rest, and their
// softmax states (the same combination rule as the decode split merge) meet in
// LDS at the end, so a tile that sees many keys gets twice the waves.
template <class E, int D, int G, int NW, int NQ, int NB, bool SPLIT, int KS>
__global__ __launch_bounds__(KS * NW * kWave, 4) void prefill_kernel(PrefillParams p) {
    using SH = PrefillShape<E, D, G, NW, NQ, NB, KS>;
    using OPS = MfmaOps<E>;
    using op4_t = typename OPS::op4_t;
    using el_t = typename std::remove_reference<decltype(op4_t{}[0])>::type;
    constexpr int RB = SH::RB, CH = SH::CH, KK = SH::KK, TT = SH::TT;
    // The two buffers are separate arrays, so the compiler can tell the LDS
    // loads filling one from the reads of the other (and need not wait for
    // them before reading); the key groups' states meet in them or in a third.
    __shared__ __attribute__((aligned(16))) char lds_a[SH::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) char lds_b[SH::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) float lds_state[SH::MERGE_BYTES / 4];

    // Grid (KV head, tile rank, sequence), KV head fastest: workgroups are
    // dealt to the XCDs round-robin in launch order, so 8 consecutive ones of
    // equal work (the same tile of 8 heads) give every XCD the same mix of
    // long and short tiles; within a sequence the last tile (most keys) goes
    // first.
    const int s = blockIdx.z;
    const int kvh = blockIdx.x;
    const int Hq = p.n_q_heads;
    const int q0 = p.cu_q[s];
    const int n = p.cu_q[s + 1] - q0;
    const int L = min(max(p.context_lens[s], 0), p.max_blocks << p.block_shift);
    if (n <= 0 || n > L) return;  // an empty or impossible chunk
    const int nrows = n * G;
    const int ntiles = (nrows + SH::ROWS - 1) / SH::ROWS;
    const int tile = ntiles - 1 - (int)blockIdx.y;
    if (tile < 0) return;
    const int r0 = tile * SH::ROWS;
    const int ctx = L - n;  // tokens before the chunk
    const int wg_last_pos = ctx + (min(r0 + SH::ROWS, nrows) - 1) / G;
    const int nblk = wg_last_pos / kBlock + 1;  // 16-token tiles the workgroup reads
    const int nit = (nblk + NB - 1) / NB;

    const int tid = threadIdx.x;
    const int kg = wave_id_uniform() / NW;  // key group
    const int w = wave_id_uniform() % NW;   // row wave within the group
    const int lane = tid % kWave;
    // iterations [kb, ke) belong to this wave's key group
    const int half = KS == 1 ? nit : (nit + 1) / 2;
    const int kb = kg == 0 ? 0 : half;
    const int ke = kg == 0 ? half : nit;
    const int gq = lane / 16;  // MFMA lane coordinates
    const int jq = lane % 16;
    const int wr0 = r0 + w * SH::ROWS_W;  // this wave's first row
    const int wave_last_pos = wr0 < nrows ? ctx + (min(wr0 + SH::ROWS_W, nrows) - 1) / G : -1;

    // The softmax below needs a positive scale: a negative one moves into q's
    // sign bits (exact), and a zero one becomes the smallest normal float,
    // which leaves every weight at exactly 1 as zero would (|score| x 2^-126
    // is far below half an ulp of 1 for any 16-bit q and K).
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    const float scale_log2 = fmaxf(fabsf(p.scale_log2), 1.17549435e-38f);
    // q rows of this wave: group c, column jq is row wr0 + 16c + jq.
    Vec16 qf[NQ][KK];
    int qpos[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const int row = wr0 + 16 * c + jq;
        const bool ok = row < nrows;
        const int tok = row / G;
        qpos[c] = ok ? ctx + tok : -1;
        const char* qrow = static_cast<const char*>(p.q) +
                           (((int64_t)(q0 + tok) * Hq + kvh * G + row % G) * D) * 2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qf[c][kk] = ok ? load16(qrow + (4 * kk + gq) * 16) : Vec16{{0u, 0u, 0u, 0u}};
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[c][kk].w[e] ^= qsign;
        }
    }
    float m[NQ], l[NQ];
    f32x4_t acc[NQ][TT];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        m[c] = -INFINITY;
        l[c] = 0.f;
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[c][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // K and V go from memory straight into LDS (buffer loads with an LDS
    // destination).  One such instruction of a wave fills a contiguous 1 KiB
    // of LDS, lane i bytes 16i .. 16i+15: RPR rows of one 16-token tile of one
    // cache, which lie in one cache block whatever the block size (RPR divides
    // 8).  Lane i fetches the global chunk that the row's XOR swizzle puts in
    // its slot.  The block's base address and the bytes of its rows inside the
    // sequence make the buffer resource, so rows past the context and invalid
    // table entries arrive as zeros (out-of-range buffer reads return 0).
    const uint32_t row_stride = (uint32_t)p.n_kv_heads * RB;
    const int bshift = p.block_shift;
    const int bsize = 1 << bshift;
    const int64_t blk_bytes = (int64_t)row_stride << bshift;
    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * RB;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * RB;
    const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks;
    constexpr int RPR = 1024 / RB;           // rows per load instruction
    constexpr int RG = kBlock / RPR;         // load instructions per tile and cache
    constexpr int PER_W = 2 * NB * RG / NW;  // load instructions per wave and iteration
    constexpr int STEP = NB * kBlock;        // tokens per iteration
    static_assert(RPR * RB == 1024 && 8 % RPR == 0 && STEP % 64 == 0 && (2 * NB * RG) % NW == 0,
                  "whole 1 KiB slices inside one block of 8 to 64, the same count per wave");
    // Slice g = w + k NW of an iteration: cache g / (NB RG), tile (g / RG) % NB,
    // rows RPR (g % RG) ..  An iteration spans a whole number of blocks, so
    // the slice's row offset inside its block is the same in every iteration
    // and goes into the lane offsets; the load's resource starts at the block
    // and covers its rows inside the sequence.
    int tok0[PER_W];   // first token of slice k in iteration 0
    int tokb0[PER_W];  // first token of its block
    uint32_t voff[PER_W];
#pragma unroll
    for (int k = 0; k < PER_W; ++k) {
        const int g = w + k * NW;
        tok0[k] = ((g / RG) % NB) * kBlock + (g % RG) * RPR;
        tokb0[k] = tok0[k] & -bsize;
        const int row = (g % RG) * RPR + lane / CH;  // row in the tile
        voff[k] = (uint32_t)(tok0[k] - tokb0[k] + lane / CH) * row_stride + (uint32_t)(((lane % CH) ^ (row % CH)) * 16);
    }
    // slices past the workgroup's last tile, or past the sequence's last table entry, load nothing
    const int tok_lim = min(nblk * kBlock, (L + bsize - 1) & -bsize);
    // LDS tiles of this key group in buffer BUF: [K, V][block][row][RB]
    auto tiles = [&](auto bufc, int kv) {
        return (decltype(bufc)::value ? lds_b : lds_a) + (kg * 2 + kv) * SH::SPAN;
    };
    // Table entries are read one step ahead of their loads: the step barrier's
    // wait covers them, and no wait for them lands behind an LDS load.
    auto entries = [&](int it, int (&pbs)[PER_W]) {
#pragma unroll
        for (int k = 0; k < PER_W; ++k) {
            const int tok = it * STEP + tok0[k];
            pbs[k] = tok < tok_lim ? table[tok >> bshift] : -1;
        }
    };
    auto issue = [&](int it, const int (&pbs)[PER_W], auto buf) {
#pragma unroll
        for (int k = 0; k < PER_W; ++k) {
            const int g = w + k * NW;  // uniform over the wave
            const int kv = g / (NB * RG), nb = (g / RG) % NB;
            const int pb = __builtin_amdgcn_readfirstlane(pbs[k]);
            const bool ok = pb >= 0 && pb < p.num_blocks;
            const int rows = min(max(L - (it * STEP + tokb0[k]), 0), bsize);  // rows of the block in the sequence
            // the size is uniform already; readfirstlane keeps the resource in scalar registers
            lds_load_1k((kv ? vbase : kbase) + (ok ? (int64_t)pb * blk_bytes : 0), ok ? (int)(rows * row_stride) : 0,
                        tiles(buf, kv) + nb * SH::TILE + (g % RG) * 1024, voff[k]);
        }
    };

    // One iteration of one wave; MASK builds the prefix-causal mask into the
    // score products' initial value (0, or -inf for a key past the row's
    // position), else every key of the iteration is visible to every row.
    auto compute = [&](auto masked, auto buf, int it) {
        constexpr bool MASK = decltype(masked)::value;
        const int b0 = it * NB;
        if (b0 * kBlock <= wave_last_pos) {
            const char* kl = tiles(buf, 0);
            const char* vl = tiles(buf, 1);
            // scores: lane (gq, jq) holds keys (b0 + nb) * 16 + 4gq + r of row column jq
            f32x4_t sacc[NQ][NB];
            if constexpr (!MASK) {
#pragma unroll
                for (int c = 0; c < NQ; ++c)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) sacc[c][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const int lim = qpos[c] - b0 * kBlock - 4 * gq;  // last visible key offset of this lane
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) sacc[c][nb][r] = 16 * nb + r <= lim ? 0.f : -INFINITY;
                }
            }
            // Every block of a computed iteration gets its products, those
            // past the wave's rows included (their scores stay -inf from the
            // mask): a branch around them would put the softmax's first reads
            // of a product's result right after it, closer than its latency.
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                Vec16 ka[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) ka[kk] = lds_load16(kl + nb * SH::TILE, tile_pos<RB>(jq, 4 * kk + gq));
#pragma unroll
                for (int c = 0; c < NQ; ++c)
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) sacc[c][nb] = OPS::qk(ka[kk], qf[c][kk], sacc[c][nb]);
            }
            op4_t ph[NQ][NB], pl[NQ][NB];
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                float mx = -INFINITY;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[c][nb][r]);
                mx = rows_max(mx);
                const float mn = mx * scale_log2;  // the row's largest scaled score here
                // The reference m[c] moves only when a row's scores pass it by
                // more than kLazy (log2 units), so the weights stay below 2^kLazy
                // and most iterations skip the rescale.
                if (__builtin_amdgcn_ballot_w64(mn > m[c] + kLazy)) {
                    const float nm = fmaxf(m[c], mn);
                    const float alpha = __builtin_amdgcn_exp2f(m[c] - (nm == -INFINITY ? 0.f : nm));
                    l[c] *= alpha;
#pragma unroll
                    for (int t = 0; t < TT; ++t) acc[c][t] *= alpha;
                    m[c] = nm;
                }
                const float ms = m[c] == -INFINITY ? 0.f : m[c];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[c][nb][r], scale_log2, -ms));
                        l[c] += pr;
                        short hs, ls;
                        OPS::split(pr, hs, ls);
                        ph[c][nb][r] = __builtin_bit_cast(el_t, hs);
                        pl[c][nb][r] = __builtin_bit_cast(el_t, ls);
                    }
            }
            // V^T read transposed: lane (gq, jq) takes key row 4gq + jq/4, bytes 32t + 8(jq%4).
            // Blocks nb and nb + 1 make one 16x16x32 product: contraction
            // slots 0-3 are keys 4gq + r of block nb, slots 4-7 those of
            // block nb + 1, in V^T and P^T alike.  A block past the wave's
            // last position has P = 0 (masked) and finite V (loaded, or zero).
            const int trow = 4 * gq + jq / 4;
#pragma unroll
            for (int nb = 0; nb < NB; nb += 2) {
                if ((b0 + nb) * kBlock > wave_last_pos) continue;
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const uint32_t off = tile_pos<RB>(trow, 2 * t + (jq % 4) / 2) + 8 * (jq % 2);
                    const op4_t a0 = OPS::read_tr(vl + nb * SH::TILE + off);
                    const op4_t a1 = OPS::read_tr(vl + (nb + 1) * SH::TILE + off);
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        acc[c][t] = OPS::pv2(a0, a1, ph[c][nb], ph[c][nb + 1], acc[c][t]);
                        if constexpr (SPLIT) acc[c][t] = OPS::pv2(a0, a1, pl[c][nb], pl[c][nb + 1], acc[c][t]);
                    }
                }
            }
        }
    };

    // Both groups step together (the barrier is the workgroup's); a group
    // whose range is shorter idles through its last step.
    // Step j computes from buffer j % 2 while the next iteration's loads fill
    // the other; they land before the step's barrier (vmcnt 0).
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    int pbs[PER_W];
    if (kb < ke) {
        entries(kb, pbs);
        issue(kb, pbs, B0{});
        if (kb + 1 < ke) entries(kb + 1, pbs);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step = [&](auto masked, int j, auto buf) {
        const int it = kb + j;
        if (it + 1 < ke) {  // uniform over the group
            issue(it + 1, pbs, std::integral_constant<int, 1 - decltype(buf)::value>{});
            if (it + 2 < ke) entries(it + 2, pbs);
        }
        if (it < ke) compute(masked, buf, it);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // Steps whose iterations (in both groups) hold only keys every row of the
    // tile sees run without the mask (an even number of them, so that the
    // buffers stay fixed per unrolled step); the rest, the causal diagonal,
    // with it.
    const int it_full = (ctx + r0 / G + 1) / (NB * kBlock);
    const int j_full = (KS == 1 ? min(it_full, half) : min(max(it_full - half, 0), half)) & ~1;
    int j = 0;
    for (; j < j_full; j += 2) {
        step(std::false_type{}, j, B0{});
        step(std::false_type{}, j + 1, B1{});
    }
    for (; j < half; j += 2) {
        step(std::true_type{}, j, B0{});
        if (j + 1 < half) step(std::true_type{}, j + 1, B1{});
    }

    // Each lane summed its own 4 keys per block: add the other lane groups.
#pragma unroll
    for (int c = 0; c < NQ; ++c) l[c] = rows_sum(l[c]);
    if constexpr (KS == 2) {
        // Group 1 leaves its state in LDS (the tiles are no longer read: the
        // loop ended on a barrier); group 0 folds it into its own.  Lane-major
        // layout, so each store and load is one conflict-free row of 64 words.
        // State element e of row group c: acc[t][r] at e = 4t + r, then m, l.
        auto slot = [&](int c, int e) -> float* {
            if constexpr (SH::STATE_IN_BUFFERS) {
                constexpr int SB = SH::STATE - SH::STATE_A;
                return e < SH::STATE_A
                           ? reinterpret_cast<float*>(lds_a) + ((w * NQ + c) * SH::STATE_A + e) * kWave + lane
                           : reinterpret_cast<float*>(lds_b) + ((w * NQ + c) * SB + e - SH::STATE_A) * kWave + lane;
            } else {
                return lds_state + ((w * NQ + c) * SH::STATE + e) * kWave + lane;
            }
        };
        if (kg == 1) {
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) *slot(c, 4 * t + r) = acc[c][t][r];
                *slot(c, 4 * TT) = m[c];
                *slot(c, 4 * TT + 1) = l[c];
            }
        }
        __syncthreads();
        if (kg == 1) return;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const float m1 = *slot(c, 4 * TT);
            const float l1 = *slot(c, 4 * TT + 1);
            const float mm = fmaxf(m[c], m1);
            const float mr = mm == -INFINITY ? 0.f : mm;
            const float a0 = __builtin_amdgcn_exp2f(m[c] - mr);
            const float a1 = __builtin_amdgcn_exp2f(m1 - mr);
            l[c] = l[c] * a0 + l1 * a1;
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[c][t][r] = acc[c][t][r] * a0 + *slot(c, 4 * t + r) * a1;
        }
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const int row = wr0 + 16 * c + jq;
        if (row >= nrows) continue;
        const float inv = 1.f / l[c];
        char* orow = static_cast<char*>(p.out) + (((int64_t)(q0 + row / G) * Hq + kvh * G + row % G) * D) * 2;
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) E::store(orow + (16 * t + 4 * gq + r) * 2, acc[c][t][r] * inv);
    }
}

template <class E, int D, int G, int NW, int NQ, int NB, bool SPLIT, int KS>
hipError_t launch_prefill_shape(const PrefillParams& p, hipStream_t stream) {
    constexpr int ROWS = NW * 16 * NQ;
    const int64_t tiles = ((int64_t)p.max_q_len * G + ROWS - 1) / ROWS;
    if (tiles > kMaxPrefillTiles || p.num_seqs > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid(p.n_kv_heads, (unsigned)tiles, (unsigned)p.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<E, D, G, NW, NQ, NB, SPLIT, KS>), grid, dim3(KS * NW * kWave), 0, stream, p);
    return hipGetLastError();
}

// Launch shape (measured on MI355X): 8 waves of 16 query rows (128 rows per
// workgroup) in each of 2 key groups; 4 blocks (64 keys) per iteration, i.e.
// 32 KiB (head_dim 128) or 16 KiB (64) of K and V per group and LDS buffer.  It
// needs no accumulator registers beyond the architectural VGPRs and runs 4
// waves per SIMD.  fp16 keeps one 16-bit P per weight (11 significant bits);
// bf16 splits P into high and low parts, since one bf16 keeps only 8.
template <class E, int D, int G>
static hipError_t launch_prefill_g(const PrefillParams& p, hipStream_t stream) {
    constexpr bool SPLIT = std::is_same<E, BF16>::value;
    static_assert(8 * 16 == kPrefillRows, "the grid's tile height");
    return launch_prefill_shape<E, D, G, 8, 1, 4, SPLIT, 2>(p, stream);
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
