// decode.hip -- paged decode attention on gfx950: the split-K pass, in two
// schedules, and the log-sum-exp merge.
//
// What is computed: for sequence s, query head h, KV head g = h / G
// (G = n_q_heads / n_kv_heads) and L = context_lens[s],
//     out[s][h] = sum_{i<L} softmax_i(scale * <q[s][h], K_i>) V_i
// where K_i, V_i are row (i mod B) of physical block block_table[s][i / B]
// ("How a serving engine actually works", paperfordummies.in, "The one
// formula"; the attention maths is unchanged by paging -- henryhe.ai,
// "What's deliberately still missing").
//
// The unit of work is a tile: one 16-token block of one KV head of one
// sequence, i.e. 16 K rows and 16 V rows of head_dim elements (rows are
// n_kv_heads * head_dim elements apart in the cache).  A wave streams tiles:
//   * loads: 16-byte nontemporal loads, R lanes per row, so one load
//     instruction reads 64/R rows x 16R contiguous bytes; the tiles of the
//     next DEPTH blocks are in flight while one is computed;
//   * the G query heads sharing KV head g reuse every K/V register tile, so
//     each K/V byte leaves HBM once per step;
//   * QK: packed 16-bit dot products with fp32 accumulation (v_dot2), summed
//     over the R lanes of a row with DPP; scores are kept in base-2 units
//     (scale * log2 e folded in) so the softmax uses v_exp_f32 directly;
//   * online softmax per row group of lanes: running max m, sum l and the
//     unnormalised accumulator acc; acc is rescaled only when some lane's max
//     grows; rows past L (last block only) are masked by select, values too,
//     so whatever those slots hold (NaN included) never reaches the output.
// A run of consecutive tiles of one (sequence, KV head) -- a segment -- ends
// with the row groups combined by the log-sum-exp rule; the segment's state
// is then either the whole answer (normalised, rounded to the cache dtype
// and written to out) or a partial record for the merge pass:
//     M = max_j m_j,  out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j.
//
// Two schedules:
//   * flat (the default): a persistent grid of W waves deals the flat stream
//     of all tiles -- ordered by sequence, KV head, block -- into W equal
//     contiguous ranges, so every wave does the same number of tiles whatever
//     the length mix.  Segments are cut where a range ends; segment (pair j,
//     wave w) keeps its record at index j + w, unique because j + w grows by
//     at least one from one segment to the next.  With the matrix-core engine
//     the unit is a team: up to 8 waves of a workgroup, one KV head each,
//     walking the same blocks in lockstep (the stream is then ordered by
//     sequence, block of team heads, block).
//   * fixed partitions (P tokens each): every partition of every (sequence,
//     head group) is computed on its own and writes its record (or the
//     output, for a sequence with one partition); a workgroup per (sequence,
//     query head) merges the records.  The matrix-core engine runs a
//     persistent grid over balanced ranges of (sequence, partition, team)
//     units, each partition split between two key groups that meet in LDS,
//     records staged in LDS and written four at a time; the vector engine,
//     and batches whose unit prefix does not fit LDS, run one workgroup per
//     NW partitions.  Both give the same bits.
//
// Everything is bound by HBM bandwidth: each (token, KV head) costs
// 2 * head_dim * element bytes of reads and 4 * head_dim * G flops.
#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_mfma.h"

namespace pkv {

// Launch shape: NW waves per workgroup, R lanes per K/V row, DEPTH tiles in
// flight ahead of the one being computed, streaming (nontemporal) loads; the
// flat schedule's grid holds at most CAP workgroups per CU (0: as many as fit);
// teams of up to TEAM waves of a workgroup walk the same blocks in lockstep,
// each wave its own head group (TEAM divides NW; 1: every wave on its own).
template <int NW_, int R_, int DEPTH_, bool STREAM_, bool MFMA_ = false, int NH_ = 1, int CAP_ = 0, int TEAM_ = 1,
          int KS_ = 1>
struct Tune {
    static constexpr int NW = NW_;
    static constexpr int R = R_;
    static constexpr int DEPTH = DEPTH_;
    static constexpr bool STREAM = STREAM_;
    static constexpr bool MFMA = MFMA_;  // matrix-core engine (16-bit caches, G >= 4)
    static constexpr int NH = NH_;       // adjacent KV heads per wave (VALU engine)
    static constexpr int CAP = CAP_;     // flat grid: workgroups per CU at most (0: occupancy)
    static constexpr int TEAM = TEAM_;   // largest team (a power of two dividing NW)
    static constexpr int KS = KS_;       // fixed partitions: waves that split one partition's tiles
    static_assert(TEAM >= 1 && (TEAM & (TEAM - 1)) == 0 && NW % (TEAM * KS) == 0, "team size");
};

// The team size for ng head groups: the largest power of two up to TU::TEAM
// that divides ng (so every team is whole).
template <class TU>
static int team_size(int ng) {
    int ts = TU::TEAM;
    while (ts > 1 && ng % ts != 0) ts /= 2;
    return ts;
}

// a ? x : y for addresses, as a select of the two values (no branch around the
// load that uses it).
__device__ __forceinline__ const char* pick(bool a, const char* x, const char* y) {
    const uint64_t ux = reinterpret_cast<uint64_t>(x), uy = reinterpret_cast<uint64_t>(y);
    return reinterpret_cast<const char*>(a ? ux : uy);
}

// One wave's share of the attention for NH adjacent KV heads (a head group)
// and the G query heads of each.  The NH head rows of one token are adjacent
// in the cache, so one load instruction reads RPS tokens x NH * RB contiguous
// bytes; lane l serves head hd = (l mod NH*R) / R only, so the per-lane state
// does not grow with NH.
template <class E, int D, int G, class TU>
struct WaveAttn {
    static constexpr int NH = TU::NH;         // KV heads per wave
    static constexpr int HG = NH * G;         // query heads per wave
    static constexpr int VEC = E::kPerVec;    // elements per 16-byte vector
    static constexpr int RB = D * E::kBytes;  // bytes per (token, head) row
    static constexpr int CH = RB / 16;        // 16-byte chunks per row
    static constexpr int R = TU::R;           // lanes sharing one head row
    static constexpr int HR = NH * R;         // lanes sharing one token's head-group row
    static constexpr int CPL = CH / R;        // chunks per lane per row
    static constexpr int RPS = kWave / HR;    // tokens covered by one load instruction
    static constexpr int J = kBlock / RPS;    // rows per lane per tile
    static constexpr int EPL = CPL * VEC;     // elements per lane per row
    static constexpr int NS = TU::DEPTH + 1;  // register tile slots
    static constexpr int kLdsBytes = 0;       // per wave
    static_assert(CH % R == 0 && kWave % HR == 0 && kBlock % RPS == 0 && J >= 1 && R <= 16, "lane mapping");

    int rg, c, hd;  // row group, chunk column and head (within the group) of this lane
    uint32_t lane_off[J][CPL];
    Vec16 qv[G][CPL];
    float acc[G][EPL];
    float m[G], l[G];
    Vec16 kb[NS][J][CPL], vb[NS][J][CPL];

    __device__ __forceinline__ void init(int lane, uint32_t row_stride, char*) {
        rg = lane / HR;
        hd = (lane % HR) / R;
        c = lane % R;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int k = 0; k < CPL; ++k)
                lane_off[j][k] = (j * RPS + rg) * row_stride + hd * RB + (c + k * R) * 16;
    }

    // q rows of the group's HG query heads (contiguous [HG][D]); this lane
    // loads its own head's G rows, its chunks only.
    __device__ __forceinline__ void load_q(const char* q_rows) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int k = 0; k < CPL; ++k) qv[gi][k] = load16(q_rows + (hd * G + gi) * RB + (c + k * R) * 16);
    }

    __device__ __forceinline__ void settle_q() const {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int k = 0; k < CPL; ++k) settle(qv[gi][k]);
    }

    // The flat schedule loads the q rows of a segment's pair into the slot of
    // the segment's first tile, right before that tile's K/V loads, so the
    // wait for the tile covers them; take_q makes them current.  Only when the
    // extra q sets are few registers (kQAhead); otherwise q is loaded where a
    // segment starts, and waited for there.
    static constexpr bool kQAhead = NS * G * CPL * 4 <= 32;
    Vec16 qs[kQAhead ? NS : 1][G][CPL];
    __device__ __forceinline__ void load_q_slot(int slot, const char* q_rows) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int k = 0; k < CPL; ++k)
                qs[slot][gi][k] = load16(q_rows + (hd * G + gi) * RB + (c + k * R) * 16);
    }
    __device__ __forceinline__ void take_q(int slot) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int k = 0; k < CPL; ++k) qv[gi][k] = qs[slot][gi][k];
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            m[gi] = -INFINITY;
            l[gi] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[gi][e] = 0.f;
        }
    }

    // Loads of one tile: row r of head g at kbase/vbase + (r < 8 ? lo : hi) + r * row_stride.
    // A load instruction covers RPS consecutive rows, all in the same half.
    // Tile row `prow` (if 0..15) is read from the rows kn, vn ([NH][D] of the
    // token being appended) instead of the cache.
    // FRESH = false: no row comes from kn / vn (prow is ignored).
    template <bool FRESH>
    __device__ __forceinline__ void issue(int slot, const char* kbase, const char* vbase, int64_t lo, int64_t hi,
                                          int prow, const char* kn, const char* vn) {
        static_assert(8 % RPS == 0, "a load instruction stays within one half of the tile");
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t boff = j * RPS < 8 ? lo : hi;
            const bool fresh = FRESH && j * RPS + rg == prow;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const uint32_t col = hd * RB + (c + k * R) * 16;
                kb[slot][j][k] = load16_policy<TU::STREAM>(pick(fresh, kn + col, kbase + boff + lane_off[j][k]));
                vb[slot][j][k] = load16_policy<TU::STREAM>(pick(fresh, vn + col, vbase + boff + lane_off[j][k]));
            }
        }
    }

    // Online-softmax update with one tile; `valid` rows (wave-uniform) belong
    // to the sequence, the rest are masked.
    __device__ __forceinline__ void process(int slot, int valid, float scale_log2) {
        float sc[G][J];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                float d = 0.f;
#pragma unroll
                for (int k = 0; k < CPL; ++k) d = E::dot(qv[gi][k], kb[slot][j][k], d);
                sc[gi][j] = group_sum<R>(d) * scale_log2;
            }
        const bool masked = valid < kBlock;  // wave-uniform: the last tile, or a skipped one
        if (masked) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int gi = 0; gi < G; ++gi) sc[gi][j] = j * RPS + rg < valid ? sc[gi][j] : -INFINITY;
        }
        float pj[G][J];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float mx = sc[gi][0];
#pragma unroll
            for (int j = 1; j < J; ++j) mx = fmaxf(mx, sc[gi][j]);
            const float mn = fmaxf(m[gi], mx);
            const float ms = mn == -INFINITY ? 0.f : mn;  // all masked so far: p = 0
            if (__builtin_amdgcn_ballot_w64(mn > m[gi])) {
                const float alpha = __builtin_amdgcn_exp2f(m[gi] - ms);
                l[gi] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[gi][e] *= alpha;
                m[gi] = mn;
            }
#pragma unroll
            for (int j = 0; j < J; ++j) {
                pj[gi][j] = __builtin_amdgcn_exp2f(sc[gi][j] - ms);
                l[gi] += pj[gi][j];
            }
        }
        // P.V, one row at a time: a row past `valid` contributes nothing, even
        // when its slot holds NaN (select, not multiply).
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const bool ok = !masked || j * RPS + rg < valid;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float vf[VEC];
                E::expand(vb[slot][j][k], vf);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float v = ok ? vf[e] : 0.f;
#pragma unroll
                    for (int gi = 0; gi < G; ++gi)
                        acc[gi][k * VEC + e] = __builtin_fmaf(pj[gi][j], v, acc[gi][k * VEC + e]);
                }
            }
        }
    }

    // Combine the row groups (lanes l, l+HR, l+2HR, ...): afterwards every
    // lane holds the wave's m, l and acc for its head and chunk column.
    __device__ __forceinline__ void reduce() {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float M = m[gi];
#pragma unroll
            for (int x = HR; x < kWave; x <<= 1) M = fmaxf(M, shfl_xor(M, x));
            const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[gi] - M);
            float lsum = l[gi] * f;
#pragma unroll
            for (int x = HR; x < kWave; x <<= 1) lsum += shfl_xor(lsum, x);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float a = acc[gi][e] * f;
#pragma unroll
                for (int x = HR; x < kWave; x <<= 1) a += shfl_xor(a, x);
                acc[gi][e] = a;
            }
            m[gi] = M;
            l[gi] = lsum;
        }
    }

    // A segment's state after reduce, as this lane holds it.  The flat
    // schedule keeps one finished segment's Result in registers and writes it
    // after the tile loop when it is small (kHold).
    struct Result {
        float acc[G][EPL];
        float m[G], l[G];
    };
    static constexpr bool kHold = G * (EPL + 2) <= 18;  // one query head per KV head: 10-18 registers

    // r = the combination of the states r and o of the same rows (log-sum-exp
    // rule; o may be empty: m = -inf, l = 0).
    __device__ static __forceinline__ void combine(Result& r, const Result& o) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const float M = fmaxf(r.m[gi], o.m[gi]);
            const float f0 = r.m[gi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(r.m[gi] - M);
            const float f1 = o.m[gi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o.m[gi] - M);
            r.l[gi] = f0 * r.l[gi] + f1 * o.l[gi];
#pragma unroll
            for (int e = 0; e < EPL; ++e) r.acc[gi][e] = f0 * r.acc[gi][e] + f1 * o.acc[gi][e];
            r.m[gi] = M;
        }
    }

    __device__ __forceinline__ void take(Result& r) const {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) r.acc[gi][e] = acc[gi][e];
            r.m[gi] = m[gi];
            r.l[gi] = l[gi];
        }
    }

    // Row group 0 writes the normalised rows of the HG query heads ([HG][D]
    // at out_rows) ...
    __device__ __forceinline__ void store_out(const Result& r, char* out_rows) const {
        if (rg != 0) return;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const float inv = 1.f / r.l[gi];
            const int row = hd * G + gi;
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < VEC; e += 4) {
                    const float* x = &r.acc[gi][k * VEC + e];
                    store4<E>(out_rows + (row * D + (c + k * R) * VEC + e) * E::kBytes, x[0] * inv, x[1] * inv,
                              x[2] * inv, x[3] * inv);
                }
        }
    }

    // ... or the partial record: acc [HG][D] fp32 and (m, l) [HG][2] fp32.
    __device__ __forceinline__ void store_partial(const Result& r, float* rec_acc, float* rec_ml) const {
        if (rg != 0) return;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const int row = hd * G + gi;
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<float4*>(rec_acc + row * D + (c + k * R) * VEC + e) =
                        make_float4(r.acc[gi][k * VEC + e], r.acc[gi][k * VEC + e + 1], r.acc[gi][k * VEC + e + 2],
                                    r.acc[gi][k * VEC + e + 3]);
            if (c == 0) {
                rec_ml[row * 2] = r.m[gi];
                rec_ml[row * 2 + 1] = r.l[gi];
            }
        }
    }

    // A state to and from LDS in the record's own order: acc [HG][D], then
    // (m, l) [HG][2].  Every lane reads back what it holds after reduce.
    __device__ __forceinline__ void stage(const Result& r, float* slot) const {
        store_partial(r, slot, slot + HG * D);
    }
    __device__ __forceinline__ void unstage(const float* slot, Result& r) const {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const int row = hd * G + gi;
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) r.acc[gi][k * VEC + e] = slot[row * D + (c + k * R) * VEC + e];
            r.m[gi] = slot[HG * D + row * 2];
            r.l[gi] = slot[HG * D + row * 2 + 1];
        }
    }
};

// ----------------------------------------------------------------------------
// Matrix-core engine for 16-bit caches and G >= 4.  Per tile of NH adjacent KV
// heads (16 tokens), with the wave's HG = NH * G query heads in columns
// 0..HG-1 of 16 (the rest zero padding):
//   S^T[16 tok][16]  = sum_h K_h[16][D] . Q_h^T[D][16]      (NH * D/32 MFMA 16x16x32)
//   O^T[D][16]      += sum_h V_h^T[D][16 tok] . P_h^T[16][16] (D/16 x 2 MFMA 16x16x32
//                      with two heads, D/16 with one: two 4-token halves each)
// Q_h^T holds only head h's columns, so both heads accumulate into one S^T
// and P_h^T keeps only head h's columns of P^T.  Lane l = 16 g + j holds S^T
// rows 4g..4g+3 of column j, which is exactly the B operand P^T, so the
// softmax state of query head j lives in lane column j and never moves.
// K and V are loaded with the wide coalesced pattern (each token's NH head
// rows, NH * D * 2 contiguous bytes, by NH * D / 8 lanes), written once to a
// per-wave LDS tile with the 16-byte chunks XOR-swizzled by row, and read back
// as MFMA operands: K with 16-byte reads (lane: row j, chunk 4kk + g), V
// transposed with ds_read_b64_tr_b16.  P is rounded to the 16-bit type as a
// sum hi + lo of two 16-bit values, so the product keeps ~16 bits of P.
// ----------------------------------------------------------------------------

template <class E, int D, int G, class TU>
struct MfmaAttn {
    static constexpr int NH = TU::NH;            // adjacent KV heads per wave
    static constexpr int HG = NH * G;            // query heads per wave (S^T columns used)
    static_assert(E::kBytes == 2 && HG <= 16 && D % 32 == 0, "16-bit caches, up to 16 query heads per wave");
    using OPS = MfmaOps<E>;
    using op4_t = typename OPS::op4_t;
    static constexpr int RB = D * 2;             // bytes per head row
    static constexpr int CH = RB / 16;           // 16-byte chunks per head row
    static constexpr int ROW = NH * RB;          // bytes of one token's NH head rows
    static constexpr int LPR = NH * CH;          // lanes per token row in a load
    static constexpr int RPI = kWave / LPR;      // token rows per load instruction
    static constexpr int NI = kBlock / RPI;      // load instructions per tile (each of K, V)
    static constexpr int KK = D / 32;            // QK products per head
    static constexpr int TT = D / 16;            // PV output tiles
    static constexpr int NS = TU::DEPTH + 1;     // register tile slots
    static constexpr int kTileBytes = kBlock * ROW;
    static constexpr int kLdsBytes = 2 * kTileBytes;  // per wave: the K and V of one tile
    static_assert(kWave % LPR == 0 && kBlock % RPI == 0 && CH == 4 * KK, "lane mapping");

    int g, j;          // MFMA lane coordinates
    int lrow, lhead, lchunk;  // this lane's token row (in a load), head and chunk
    char* lds;
    uint32_t ld_base;  // this lane's byte offset in a tile (first load instruction)
    Vec16 qb[NH][KK];
    f32x4_t acc[TT];
    float m, l;
    Vec16 kt[NS][NI], vt[NS][NI];

    __device__ __forceinline__ static uint32_t lds_pos(int row, int head, int chunk) {
        return (uint32_t)(row * ROW + head * RB + ((chunk ^ (row % CH)) * 16));
    }

    __device__ __forceinline__ void init(int lane, uint32_t row_stride, char* lds_wave) {
        g = lane / 16;
        j = lane % 16;
        lrow = lane / LPR;
        lhead = (lane % LPR) / CH;
        lchunk = lane % CH;
        lds = lds_wave;
        ld_base = lrow * row_stride + lhead * RB + lchunk * 16;
        row_stride_ = row_stride;
    }
    uint32_t row_stride_;

    // q rows of the wave's HG query heads (contiguous [HG][D]): column j takes
    // row j, in the B operand of head j / G only.
    __device__ __forceinline__ void load_q(const char* q_rows) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const Vec16 z = {{0u, 0u, 0u, 0u}};
                qb[h][kk] = (j >= h * G && j < (h + 1) * G) ? load16(q_rows + j * RB + (4 * kk + g) * 16) : z;
            }
    }

    __device__ __forceinline__ void settle_q() const {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) settle(qb[h][kk]);
    }

    // As in WaveAttn: a segment's q rows ride in the slot of its first tile.
    static constexpr bool kQAhead = NS * NH * KK * 4 <= 32;
    Vec16 qs[kQAhead ? NS : 1][NH][KK];
    __device__ __forceinline__ void load_q_slot(int slot, const char* q_rows) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const Vec16 z = {{0u, 0u, 0u, 0u}};
                qs[slot][h][kk] = (j >= h * G && j < (h + 1) * G) ? load16(q_rows + j * RB + (4 * kk + g) * 16) : z;
            }
    }
    __device__ __forceinline__ void take_q(int slot) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) qb[h][kk] = qs[slot][h][kk];
    }

    __device__ __forceinline__ void reset() {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Tile row `prow` (if 0..15) is read from the rows kn, vn ([NH][D] of the
    // token being appended) instead of the cache.
    template <bool FRESH>
    __device__ __forceinline__ void issue(int slot, const char* kbase, const char* vbase, int64_t lo, int64_t hi,
                                          int prow, const char* kn, const char* vn) {
        static_assert(8 % RPI == 0, "a load instruction stays within one half of the tile");
        const uint32_t col = lhead * RB + lchunk * 16;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t off = (i * RPI < 8 ? lo : hi) + ld_base + (int64_t)i * RPI * row_stride_;
            const bool fresh = FRESH && i * RPI + lrow == prow;
            kt[slot][i] = load16_policy<TU::STREAM>(pick(fresh, kn + col, kbase + off));
            vt[slot][i] = load16_policy<TU::STREAM>(pick(fresh, vn + col, vbase + off));
        }
    }

    __device__ __forceinline__ void process(int slot, int valid, float scale_log2) {
        char* kl = lds;
        char* vl = lds + kTileBytes;
        // K and V rows into LDS; V rows past `valid` are written as zeros.
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = i * RPI + lrow;
            const uint32_t pos = lds_pos(row, lhead, lchunk);
            lds_store16(kl, pos, kt[slot][i]);
            Vec16 v = vt[slot][i];
            if (valid < kBlock && row >= valid) v = Vec16{{0u, 0u, 0u, 0u}};
            lds_store16(vl, pos, v);
        }
        // the rows this wave just stored are read back by other lanes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // two accumulators, so the score products form two chains half as long
        f32x4_t sacc0 = {0.f, 0.f, 0.f, 0.f}, sacc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const Vec16 ka = lds_load16(kl, lds_pos(j, h, 4 * kk + g));
                if ((h * KK + kk) % 2 == 0) sacc0 = OPS::qk(ka, qb[h][kk], sacc0);
                else sacc1 = OPS::qk(ka, qb[h][kk], sacc1);
            }
        const f32x4_t sacc = sacc0 + sacc1;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sc[r] = sacc[r] * scale_log2;
            if (valid < kBlock && 4 * g + r >= valid) sc[r] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = rows_max(mx);
        const float mn = fmaxf(m, mx);
        const float ms = mn == -INFINITY ? 0.f : mn;
        if (__builtin_amdgcn_ballot_w64(mn > m)) {
            const float alpha = __builtin_amdgcn_exp2f(m - ms);
            l *= alpha;
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[t] *= alpha;
            m = mn;
        }
        op4_t phi, plo;
        using el_t = typename std::remove_reference<decltype(phi[0])>::type;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = __builtin_amdgcn_exp2f(sc[r] - ms);
            l += pr;
            short h, lo;
            OPS::split(pr, h, lo);
            phi[r] = __builtin_bit_cast(el_t, h);
            plo[r] = __builtin_bit_cast(el_t, lo);
        }
        const op4_t zero = {};
        // V^T read transposed: lane (g, j) takes row 4g + j/4, bytes 32t + 8(j%4) of its head row.
        // Each 16x16x32 product takes two 4-token halves: with two heads, head
        // 0's V^T and P^T beside head 1's (a column's P is zero for the head it
        // does not belong to); with one head, V^T twice beside P's high and
        // low parts.
        const int trow = 4 * g + j / 4;
        if constexpr (NH == 2) {
            const bool m0 = j < G, m1 = j >= G && j < 2 * G;
            const op4_t bh0 = m0 ? phi : zero, bl0 = m0 ? plo : zero;
            const op4_t bh1 = m1 ? phi : zero, bl1 = m1 ? plo : zero;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const uint32_t off = 2 * t + (j % 4) / 2;
                const op4_t a0 = OPS::read_tr(vl + lds_pos(trow, 0, off) + 8 * (j % 2));
                const op4_t a1 = OPS::read_tr(vl + lds_pos(trow, 1, off) + 8 * (j % 2));
                acc[t] = OPS::pv2(a0, a1, bh0, bh1, acc[t]);
                acc[t] = OPS::pv2(a0, a1, bl0, bl1, acc[t]);
            }
        } else {
            static_assert(NH == 1, "one or two KV heads per wave");
            const bool mine = j < G;
            const op4_t bh = mine ? phi : zero, bl = mine ? plo : zero;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const op4_t a = OPS::read_tr(vl + lds_pos(trow, 0, 2 * t + (j % 4) / 2) + 8 * (j % 2));
                acc[t] = OPS::pv2(a, a, bh, bl, acc[t]);
            }
        }
    }

    __device__ __forceinline__ void reduce() {
        l = rows_sum(l);
    }

    // A segment's state after reduce (see WaveAttn::Result).
    struct Result {
        f32x4_t acc[TT];
        float m, l;
    };
    static constexpr bool kHold = HG <= 4;  // more query heads leave no registers to spare

    // r = the combination of r and o (see WaveAttn::combine).
    __device__ static __forceinline__ void combine(Result& r, const Result& o) {
        const float M = fmaxf(r.m, o.m);
        const float f0 = r.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(r.m - M);
        const float f1 = o.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o.m - M);
        r.l = f0 * r.l + f1 * o.l;
#pragma unroll
        for (int t = 0; t < TT; ++t) r.acc[t] = f0 * r.acc[t] + f1 * o.acc[t];
        r.m = M;
    }

    __device__ __forceinline__ void take(Result& r) const {
#pragma unroll
        for (int t = 0; t < TT; ++t) r.acc[t] = acc[t];
        r.m = m;
        r.l = l;
    }

    __device__ __forceinline__ void store_out(const Result& r, char* out_rows) const {
        if (j >= HG) return;
        const float inv = 1.f / r.l;
#pragma unroll
        for (int t = 0; t < TT; ++t)
            store4<E>(out_rows + (j * D + 16 * t + 4 * g) * 2, r.acc[t][0] * inv, r.acc[t][1] * inv,
                      r.acc[t][2] * inv, r.acc[t][3] * inv);
    }

    __device__ __forceinline__ void store_partial(const Result& r, float* rec_acc, float* rec_ml) const {
        if (j >= HG) return;
#pragma unroll
        for (int t = 0; t < TT; ++t)
            *reinterpret_cast<float4*>(rec_acc + j * D + 16 * t + 4 * g) =
                make_float4(r.acc[t][0], r.acc[t][1], r.acc[t][2], r.acc[t][3]);
        if (g == 0) {
            rec_ml[j * 2] = r.m;
            rec_ml[j * 2 + 1] = r.l;
        }
    }

    // See WaveAttn::stage; columns past HG (padding) read back as empty states.
    __device__ __forceinline__ void stage(const Result& r, float* slot) const {
        store_partial(r, slot, slot + HG * D);
    }
    __device__ __forceinline__ void unstage(const float* slot, Result& r) const {
        if (j >= HG) {
#pragma unroll
            for (int t = 0; t < TT; ++t) r.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            r.m = -INFINITY;
            r.l = 0.f;
            return;
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float4 v = *reinterpret_cast<const float4*>(slot + j * D + 16 * t + 4 * g);
            r.acc[t] = f32x4_t{v.x, v.y, v.z, v.w};
        }
        r.m = slot[HG * D + j * 2];
        r.l = slot[HG * D + j * 2 + 1];
    }
};

template <class E, int D, int G, class TU>
using Engine = typename std::conditional<TU::MFMA, MfmaAttn<E, D, G, TU>, WaveAttn<E, D, G, TU>>::type;

// Where tile t (tokens 16t .. 16t+15) of a sequence lives.  The table row lists
// ntab blocks of B = 1 << shift tokens (B in {8, 16, 32, 64}); rows 0-7 of the
// tile are at lo + r * row_stride and rows 8-15 at hi + r * row_stride.  With
// B >= 16 the tile lies inside one block (hi = lo); with B = 8 it spans two,
// and a second block past the sequence (whose rows are masked) is replaced by
// rows 0-7 of the first.  ok is false if a block the tile needs lies outside
// the pool; the offsets then point at block 0, inside the cache.
struct TileAddr {
    int64_t lo, hi;
    bool ok;
};

// Loads issued past the end of a wave's tiles read rows 0-7 of block 0 twice
// (lo = 0, hi = -8 rows): inside the cache at every block size.
constexpr int kDummyRows = 8;

// A table entry is read with a scalar load: the table is constant while the
// kernel runs and the wave's index is uniform, so the read goes through the
// constant address space.  A vector load would be counted together with the
// K/V loads in flight, and waiting for its value would wait for all of them.
typedef const __attribute__((address_space(4))) int32_t const_i32;

__device__ __forceinline__ int table_entry(const int32_t* table, int i) {
    return ((const_i32*)table)[__builtin_amdgcn_readfirstlane(i)];
}

// The table entries tile t needs: the block of rows 0-7 and, when B = 8 and
// the second block belongs to the sequence, the block of rows 8-15.
struct TileEnt {
    int pb0, pb1;
};

__device__ __forceinline__ TileEnt tile_entries(const int32_t* table, int t, int ntab, int shift) {
    const int tok0 = t * kBlock;
    const int bi0 = tok0 >> shift;
    const int bi1 = (tok0 + 8) >> shift;
    const bool second = bi1 != bi0 && bi1 < ntab;
    TileEnt e;
    e.pb0 = table_entry(table, bi0);
    e.pb1 = table_entry(table, second ? bi1 : bi0);  // no branch: neither read waits here
    return e;
}

__device__ __forceinline__ TileAddr tile_addr_of(TileEnt e, int t, int ntab, int shift, int num_blocks,
                                                 uint32_t row_stride) {
    const int tok0 = t * kBlock;
    const int bmask = (1 << shift) - 1;
    const int64_t blk_bytes = (int64_t)row_stride << shift;
    const int bi0 = tok0 >> shift;
    const int bi1 = (tok0 + 8) >> shift;
    const bool second = bi1 != bi0 && bi1 < ntab;
    int pb0 = e.pb0;
    int pb1 = e.pb1;
    TileAddr a;
    a.ok = pb0 >= 0 && pb0 < num_blocks && pb1 >= 0 && pb1 < num_blocks;
    if (!a.ok) pb0 = pb1 = 0;
    a.lo = (int64_t)pb0 * blk_bytes + (int64_t)(tok0 & bmask) * row_stride;
    if (bi1 == bi0) a.hi = a.lo;
    else if (second) a.hi = (int64_t)pb1 * blk_bytes - 8 * (int64_t)row_stride;
    else a.hi = a.lo - 8 * (int64_t)row_stride;
    return a;
}

__device__ __forceinline__ TileAddr tile_addr(const int32_t* table, int t, int ntab, int shift, int num_blocks,
                                              uint32_t row_stride) {
    return tile_addr_of(tile_entries(table, t, ntab, shift), t, ntab, shift, num_blocks, row_stride);
}

// ============================================================================
// Staged results.  A finished piece of work (the state of HG query heads) can
// wait in LDS and be written later with the others: a store is counted with
// the loads in flight, and under the read traffic its acknowledgement takes
// longer than a tile, so every wait after a store in the tile loop stalls.
// Slot: acc [HG][D], (m, l) [HG][2], then the destination: kind (0: a partial
// record at index dst, 1: normalised output rows from row dst), dst low and
// high words, one word of padding (slots stay 16-byte aligned).
// ============================================================================

template <int D, int HG>
struct StageSlot {
    static constexpr int kFloats = HG * D + 2 * HG + 4;
};
constexpr int kPartStaged = 4;  // slots per wave of the fixed-partition kernel

__device__ __forceinline__ void stage_header(float* slot, int nfloats, bool out_rows, int64_t dst) {
    if (threadIdx.x % kWave == 0) {
        slot[nfloats - 3] = __int_as_float(out_rows ? 1 : 0);
        slot[nfloats - 2] = __uint_as_float((uint32_t)(uint64_t)dst);
        slot[nfloats - 1] = __uint_as_float((uint32_t)((uint64_t)dst >> 32));
    }
}

// Write n staged slots (one wave).  Records go out with nontemporal stores
// (acknowledged sooner under the read traffic); output rows are rounded to
// the cache type, four elements a store.
template <class E, int D, int HG>
__device__ __forceinline__ void write_staged(const float* slots, int n, const DecodeParams& p) {
    constexpr int SLOT = StageSlot<D, HG>::kFloats;
    const int lane = threadIdx.x % kWave;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the slots were written by other lanes
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int b = 0; b < n; ++b) {
        const float* sl = slots + b * SLOT;
        const int kind = __builtin_amdgcn_readfirstlane(__float_as_int(sl[SLOT - 3]));
        const uint32_t lo = __builtin_amdgcn_readfirstlane(__float_as_uint(sl[SLOT - 2]));
        const uint32_t hi = __builtin_amdgcn_readfirstlane(__float_as_uint(sl[SLOT - 1]));
        const int64_t dst = (int64_t)(((uint64_t)hi << 32) | lo);
        if (kind == 0) {
            float* ra = p.ws_acc + dst * HG * D;
            for (int i = lane * 4; i < HG * D; i += kWave * 4) {
                const v4u32_t v = *reinterpret_cast<const v4u32_t*>(sl + i);
                __builtin_nontemporal_store(v, reinterpret_cast<v4u32_t*>(ra + i));
            }
            if (lane < 2 * HG) p.ws_ml[dst * HG * 2 + lane] = sl[HG * D + lane];
        } else {
            char* o = static_cast<char*>(p.out) + dst * D * E::kBytes;
            for (int i = lane * 4; i < HG * D; i += kWave * 4) {
                const float inv = 1.f / sl[HG * D + (i / D) * 2 + 1];  // D is a multiple of 4
                const float4 v = *reinterpret_cast<const float4*>(sl + i);
                store4<E>(o + i * E::kBytes, v.x * inv, v.y * inv, v.z * inv, v.w * inv);
            }
        }
    }
}

// ============================================================================
// Flat schedule: a persistent grid deals equal ranges of the tile stream.
// ============================================================================

// The flat schedule's team offsets in a period of Q = 2 TW teams (the TW
// teams of two consecutive workgroups) of P tiles: team q takes
// [flat_offset(q), flat_offset(q + 1)).  Weights: the first workgroup of the
// pair xcd, the second 100 - xcd; in a workgroup of two teams, the first
// split and the second 100 - split, else all alike.
__device__ __forceinline__ int flat_offset(int q, int TW, int P, int split, int xcd) {
    auto in_wg = [&](int n) { return TW == 2 ? (n <= 0 ? 0 : n == 1 ? split : 100) : 50 * n; };
    const int64_t cum = (int64_t)xcd * in_wg(min(q, TW)) + (int64_t)(100 - xcd) * in_wg(max(q - TW, 0));
    const int64_t tot = (int64_t)100 * in_wg(TW);
    return (int)(P * cum / tot);
}

template <class E, int D, int G, class TU, bool FUSED, class A = Engine<E, D, G, TU>>
__global__ __launch_bounds__(TU::NW * kWave) void decode_flat_kernel(DecodeParams p) {
    constexpr int NS = A::NS;
    constexpr int DEPTH = TU::DEPTH;
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    const int S = p.num_seqs;
    const int Hkv = p.n_kv_heads;
    const int NG = Hkv / A::NH;  // head groups
    const int TS = p.team;       // waves per team (divides NG and NW)
    const int NGB = NG / TS;     // blocks of TS head groups: the tile stream's middle index
    const int Hq = p.n_q_heads;
    // [NW engine areas][Ls: clamped context length per sequence][pre: tile prefix]
    int32_t* Ls = reinterpret_cast<int32_t*>(dyn_lds + TU::NW * A::kLdsBytes);
    int32_t* pre = Ls + S;  // pre[s] = tiles of sequences < s; pre[S] = all tiles

    // Tile counts and their prefix sums (every workgroup computes them).
    const int max_len = p.max_blocks << p.block_shift;
    for (int i = threadIdx.x; i < S; i += blockDim.x) Ls[i] = min(max(p.context_lens[i], 0), max_len);
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        int carry = 0;
        for (int base = 0; base < S; base += kWave) {
            const int i = base + lane;
            int v = i < S ? ((Ls[i] + kBlock - 1) / kBlock) * NGB : 0;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int y = __shfl_up(v, off, kWave);
                if (lane >= off) v += y;
            }
            if (i < S) pre[i + 1] = carry + v;
            carry += __shfl(v, kWave - 1, kWave);
        }
        if (lane == 0) pre[0] = 0;
    }
    __syncthreads();
    const int T = pre[S];
    const int NT = gridDim.x * (TU::NW / TS);  // teams in the grid
    // The stream is dealt out in periods of Q = 2 NW / TS teams, the teams of
    // two consecutive workgroups: period j holds tiles [j P, (j + 1) P) and
    // team j Q + q takes [j P + off[q], j P + off[q + 1]) of it, off in
    // proportion to integer weights.  Waves given equal shares do not finish
    // together: workgroups are dealt to the XCDs round-robin, and the odd
    // XCDs stream more slowly than the even ones (xcd_pct: the even
    // workgroup's share of a pair); and in a workgroup of two teams of 4 the
    // second wave of each SIMD (waves 4-7) streams more slowly than the first,
    // which is older and issues first (split_pct: the first team's share).
    const int TW = TU::NW / TS;  // teams per workgroup
    const int Q = 2 * TW;
    const int per = max((T + NT - 1) / NT, p.min_tiles_per_worker);
    const int P = Q * per;
    if (blockIdx.x == 0) {  // the schedule, for the merge pass
        if (threadIdx.x == 0) {
            p.ws_hdr[0] = P;
            p.ws_hdr[1] = Q;
        }
        if ((int)threadIdx.x <= Q) p.ws_hdr[S + 3 + threadIdx.x] = flat_offset(threadIdx.x, TW, P, p.split_pct, p.xcd_pct);
        for (int i = threadIdx.x; i <= S; i += blockDim.x) p.ws_hdr[2 + i] = pre[i];
    }

    // Team `team` takes its share of the stream; its wave tj streams head
    // group hb * TS + tj of each tile (sequence, hb, block), so the team's
    // waves read the same blocks at the same time.
    const int w = blockIdx.x * TU::NW + wave_id_uniform();
    const int team = w / TS;
    const int tj = w - team * TS;
    const int t0 = min((team / Q) * P + flat_offset(team % Q, TW, P, p.split_pct, p.xcd_pct), T);
    const int t1 = min((team / Q) * P + flat_offset(team % Q + 1, TW, P, p.split_pct, p.xcd_pct), T);
    if (t0 >= t1) return;

    const int lane = threadIdx.x % kWave;
    const uint32_t row_stride = (uint32_t)Hkv * A::RB;
    const char* kcache = static_cast<const char*>(p.k_cache);
    const char* vcache = static_cast<const char*>(p.v_cache);
    // FUSED: an append in the same call (positions != nullptr).

    // Cursor over the tile stream, kept in scalar registers: sequence, block
    // of TS head groups, block, blocks and length of the sequence.
    struct Cur {
        int s, kvh, b, nb, L;
    };
    auto uniform = [](Cur& q) {
        q.s = __builtin_amdgcn_readfirstlane(q.s);
        q.kvh = __builtin_amdgcn_readfirstlane(q.kvh);
        q.b = __builtin_amdgcn_readfirstlane(q.b);
        q.nb = __builtin_amdgcn_readfirstlane(q.nb);
        q.L = __builtin_amdgcn_readfirstlane(q.L);
    };
    auto locate = [&](int t) {
        int lo = 0, hi = S;  // largest s with pre[s] <= t (then t < pre[s + 1])
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= t) lo = mid;
            else hi = mid;
        }
        Cur q;
        q.s = lo;
        q.L = Ls[lo];
        q.nb = (q.L + kBlock - 1) / kBlock;
        const int r = t - pre[lo];
        q.kvh = r / q.nb;
        q.b = r - q.kvh * q.nb;
        uniform(q);
        return q;
    };
    // Only a move to the next sequence reads LDS.
    auto advance = [&](Cur& q) {
        if (++q.b == q.nb) {
            q.b = 0;
            if (++q.kvh == NGB) {
                q.kvh = 0;
                do {
                    ++q.s;
                } while (q.s < S && Ls[q.s] == 0);
                q.L = q.s < S ? Ls[q.s] : 0;
                q.nb = q.s < S ? (q.L + kBlock - 1) / kBlock : 1;
            }
        }
        uniform(q);
    };

    A a;
    a.init(lane, row_stride, dyn_lds + wave_id_uniform() * A::kLdsBytes);
    bool oks[NS];
    const int bmask = (1 << p.block_shift) - 1;
    // The scalar reads a tile's issue needs (table entries, and the new
    // token's position when an append is fused) are made one issue ahead, so
    // their latency passes while the tile before is computed.
    struct Ahead {
        TileEnt e;
        int pos;
    };
    auto fetch = [&](const Cur& q, bool real) {
        Ahead f = {{0, 0}, -1};
        if (real) {
            const int ntab = (q.L + bmask) >> p.block_shift;
            f.e = tile_entries(p.block_tables + (int64_t)q.s * p.max_blocks, q.b, ntab, p.block_shift);
            if constexpr (FUSED) f.pos = table_entry(p.positions, q.s);
        }
        return f;
    };
    // Every pass issues its loads, also past the wave's last tile (then of the
    // first rows of block 0, never computed): loads are counted in issue order,
    // and a load issued on one path only would make the wait for the tile
    // being computed also wait for the tiles issued after it.
    int qs_s = -1, qs_k = -1;  // pair of the last tile issued
    auto issue = [&](int slot, const Cur& q, const Ahead& f, bool real) {
        if constexpr (A::kQAhead) {
            if (real && (q.s != qs_s || q.kvh != qs_k)) {  // the first tile of a segment carries its q rows
                qs_s = q.s;
                qs_k = q.kvh;
                a.load_q_slot(slot,
                              static_cast<const char*>(p.q) + ((int64_t)q.s * Hq + (q.kvh * TS + tj) * A::HG) * A::RB);
            }
        }
        TileAddr ta = {0, -kDummyRows * (int64_t)row_stride, false};
        if (real) {
            const int ntab = (q.L + bmask) >> p.block_shift;
            ta = tile_addr_of(f.e, q.b, ntab, p.block_shift, p.num_blocks, row_stride);
        }
        const int64_t hoff = real ? (int64_t)(q.kvh * TS + tj) * A::NH * A::RB : 0;
        // With an append in the same call, the tile holding the new token's
        // position reads that row from k_new / v_new.
        int prow = -1;
        const char *kn = kcache, *vn = vcache;
        if constexpr (FUSED) {
            const int r = f.pos - q.b * kBlock;
            if (real && r >= 0 && r < kBlock) {
                prow = r;
                const int64_t roff = ((int64_t)q.s * Hkv + (q.kvh * TS + tj) * A::NH) * A::RB;
                kn = static_cast<const char*>(p.k_new) + roff;
                vn = static_cast<const char*>(p.v_new) + roff;
            }
        }
        a.template issue<FUSED>(slot, kcache + hoff, vcache + hoff, ta.lo, ta.hi, prow, kn, vn);
        oks[slot] = ta.ok;
    };

    Cur cur = locate(t0);
    int as = -1, akvh = -1, aL = 0;  // the segment being accumulated (none yet)
    a.reset();

    Cur iss = cur;
    Ahead ahead = fetch(iss, t0 < t1);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        const bool real = t0 + d < t1;
        issue(d, iss, ahead, real);
        if (real) advance(iss);
        ahead = fetch(iss, t0 + d + 1 < t1);
    }

    // A finished segment is written as normalised output rows when this wave
    // held the whole pair, else as the partial record of (pair, wave).
    auto emit = [&](const typename A::Result& r, bool whole, int64_t dst) {
        if (whole) a.store_out(r, static_cast<char*>(p.out) + dst * D * E::kBytes);
        else a.store_partial(r, p.ws_acc + dst * A::HG * D, p.ws_ml + dst * A::HG * 2);
    };
    // Stores are counted together with the loads in flight, and the registers
    // that format them may still await a prefetched tile, so a store inside
    // the tile loop makes the next wait also wait for the tiles issued before
    // it.  With a small Result the wave keeps one finished segment in
    // registers and writes it after its last tile; only a third segment
    // writes the held one inside the loop.
    typename A::Result held;
    bool held_whole = false, have_held = false;
    int64_t held_dst = 0;
    auto flush = [&]() {
        a.reduce();
        const int nb = (aL + kBlock - 1) / kBlock;
        const int p0 = pre[as] + akvh * nb;  // the pair's tiles are [p0, p0 + nb)
        // the ranges are contiguous, so the pair is whole here when it lies in this team's
        const bool whole = p0 >= t0 && p0 + nb <= t1;
        // split pairs: record (pair + team) * TS + tj, unique because pair + team
        // grows by at least one from one segment of a wave to the next
        const int64_t dst = whole ? (int64_t)as * Hq + (akvh * TS + tj) * A::HG
                                  : ((int64_t)as * NGB + akvh + team) * TS + tj;
        if constexpr (A::kHold) {
            if (have_held) emit(held, held_whole, held_dst);
            a.take(held);
            held_whole = whole;
            held_dst = dst;
            have_held = true;
        } else {
            typename A::Result r;
            a.take(r);
            emit(r, whole, dst);
        }
    };

    for (int t = t0; t < t1; t += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int tt = t + u;
            const bool real = tt + DEPTH < t1;
            issue((u + DEPTH) % NS, iss, ahead, real);
            if (real) advance(iss);
            ahead = fetch(iss, tt + DEPTH + 1 < t1);
            if (tt < t1) {
                if (cur.s != as || cur.kvh != akvh) {
                    if (as >= 0) flush();
                    as = cur.s;
                    akvh = cur.kvh;
                    aL = cur.L;
                    if constexpr (A::kQAhead) {
                        a.take_q(u);
                    } else {
                        a.load_q(static_cast<const char*>(p.q) + ((int64_t)as * Hq + (akvh * TS + tj) * A::HG) * A::RB);
                        a.settle_q();  // here, not at the next product, where it would also wait for the next tiles
                    }
                    a.reset();
                }
                const int valid = !oks[u] ? 0 : (cur.b == cur.nb - 1 ? cur.L - cur.b * kBlock : kBlock);
                a.process(u, valid, p.scale_log2);
                advance(cur);
            }
        }
    }
    flush();
    if constexpr (A::kHold) emit(held, held_whole, held_dst);
}

// Log-sum-exp combination, by one wave, of n partial records: record x has its
// (m, l) at ml[(first + x * stride) * 2] and its acc row at acc[(first + x * stride) * D].
// A pair usually has a few records, so the (m, l) of records 0..63 (one per
// lane) and the acc rows of records 0..3 are loaded together, before anything
// waits: one memory round trip serves the common case.  Further acc rows are
// read UNROLL at a time.
template <class E, int D>
__device__ __forceinline__ void merge_records(const float* ml, const float* acc, int64_t first, int stride, int n,
                                              char* out_row) {
    constexpr int PER = (D + kWave - 1) / kWave;
    constexpr int UNROLL = 4;
    const int lane = threadIdx.x % kWave;
    auto load_rows = [&](int x0, int i, int cnt, float (&a)[UNROLL][PER]) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const bool ok = i + u < cnt;
            const int64_t r = first + (int64_t)(x0 + (ok ? i + u : 0)) * stride;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int d = lane + k * kWave;
                a[u][k] = (ok && d < D) ? acc[r * D + d] : 0.f;
            }
        }
    };
    float a0[UNROLL][PER];
    load_rows(0, 0, min(kWave, n), a0);
    float m0 = -INFINITY, l0 = 0.f;  // record `lane` (the first 64)
    if (lane < n) {
        const int64_t r = first + (int64_t)lane * stride;
        m0 = ml[r * 2];
        l0 = ml[r * 2 + 1];
    }
    float M = m0;
    for (int x = lane + kWave; x < n; x += kWave) M = fmaxf(M, ml[(first + (int64_t)x * stride) * 2]);
    M = wave_max(M);
    const float w0 = lane < n ? __builtin_amdgcn_exp2f(m0 - M) : 0.f;
    float den = w0 * l0;
    for (int x = lane + kWave; x < n; x += kWave) {
        const int64_t r = first + (int64_t)x * stride;
        den += __builtin_amdgcn_exp2f(ml[r * 2] - M) * ml[r * 2 + 1];
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) den += shfl_xor(den, m);
    float num[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] = 0.f;
    for (int x0 = 0; x0 < n; x0 += kWave) {
        // weights of records x0 .. x0+63, one per lane, then broadcast
        const int xl = x0 + lane;
        const float fl = x0 == 0 ? w0 : (xl < n ? __builtin_amdgcn_exp2f(ml[(first + (int64_t)xl * stride) * 2] - M) : 0.f);
        const int cnt = min(kWave, n - x0);
        for (int i = 0; i < cnt; i += UNROLL) {
            float a[UNROLL][PER], f[UNROLL];
            if (x0 == 0 && i == 0) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int k = 0; k < PER; ++k) a[u][k] = a0[u][k];
            } else {
                load_rows(x0, i, cnt, a);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) f[u] = __shfl(fl, i + u, kWave);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int k = 0; k < PER; ++k) num[k] = __builtin_fmaf(f[u], a[u][k], num[k]);
        }
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = lane + k * kWave;
        if (d < D) E::store(out_row + d * E::kBytes, num[k] * inv);
    }
}

// The append of a fused call, made once every read of the step is done: the
// new token's K and V rows of KV head kvh go to their slot.  Like the append
// kernel, a position or table entry out of range skips the sequence.
template <class E, int D>
__device__ __forceinline__ void append_head_row(const DecodeParams& p, int s, int kvh, int lane) {
    constexpr int RB = D * E::kBytes;  // a multiple of 16 bytes, at most 64 x 16
    const int pos = p.positions[s];
    if (pos < 0 || (pos >> p.block_shift) >= p.max_blocks) return;
    const int blk = p.block_tables[(int64_t)s * p.max_blocks + (pos >> p.block_shift)];
    if (blk < 0 || blk >= p.num_blocks) return;
    const int64_t slot = ((int64_t)blk << p.block_shift) + (pos & ((1 << p.block_shift) - 1));
    const int64_t dst = (slot * p.n_kv_heads + kvh) * RB + lane * 16;
    const int64_t src = ((int64_t)s * p.n_kv_heads + kvh) * RB + lane * 16;
    if (lane < RB / 16) {
        store16(static_cast<char*>(p.k_cache_w) + dst, load16(static_cast<const char*>(p.k_new) + src));
        store16(static_cast<char*>(p.v_cache_w) + dst, load16(static_cast<const char*>(p.v_new) + src));
    }
}

// One wave per (sequence, query head): combine the records of pairs that were
// split between waves, and write zeros for empty sequences.
template <class E, int D>
__global__ __launch_bounds__(256) void decode_flat_merge_kernel(DecodeParams p) {
    constexpr int PER = (D + kWave - 1) / kWave;
    const int lane = threadIdx.x % kWave;
    const int pair = blockIdx.x * (blockDim.x / kWave) + wave_id_uniform();
    if (pair >= p.num_seqs * p.n_q_heads) return;
    const int s = pair / p.n_q_heads;
    const int h = pair % p.n_q_heads;
    const int Gq = p.n_q_heads / p.n_kv_heads;
    if (p.positions != nullptr && h % Gq == 0) append_head_row<E, D>(p, s, h / Gq, lane);
    const int HG = p.n_q_heads / p.n_kv_heads * p.heads_per_wave;  // query heads per record
    const int NG = p.n_kv_heads / p.heads_per_wave;
    const int TS = p.team;
    const int NGB = NG / TS;
    const int hg = h / HG;
    const int hb = hg / TS;
    const int tj = hg - hb * TS;
    const int gi = h % HG;
    char* out_row = static_cast<char*>(p.out) + (int64_t)pair * D * E::kBytes;
    const int L = min(max(p.context_lens[s], 0), (p.max_blocks << p.block_shift));
    if (L == 0) {
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (lane + k * kWave < D) E::store(out_row + (lane + k * kWave) * E::kBytes, 0.f);
        return;
    }
    // team j Q + q holds tiles [j P + off[q], j P + off[q + 1]) (see decode_flat_kernel)
    const int S = p.num_seqs;
    const int P = p.ws_hdr[0], Q = p.ws_hdr[1];
    const int32_t* off = p.ws_hdr + S + 3;
    auto piece = [&](int t) {
        const int r = t % P;
        int q = 0;
        for (int i = 1; i < Q; ++i) q += off[i] <= r ? 1 : 0;
        return (t / P) * Q + q;
    };
    const int nb = (L + kBlock - 1) / kBlock;
    const int p0 = p.ws_hdr[2 + s] + hb * nb;
    const int w0 = piece(p0);  // teams w0 .. w1 hold the pair's tiles
    const int w1 = piece(p0 + nb - 1);
    if (w0 == w1) return;  // one wave held the whole pair and wrote it
    const int64_t base = (int64_t)s * NGB + hb;  // record of team w is (base + w) * TS + tj
    merge_records<E, D>(p.ws_ml, p.ws_acc, ((base + w0) * TS + tj) * HG + gi, TS * HG, w1 - w0 + 1, out_row);
}

// ============================================================================
// Fixed partitions: the P-token partitions of every sequence are computed
// alone (so a sequence's result does not depend on the rest of the batch),
// each by KS waves that split its tiles, one key group each, for each of its
// head groups.  A workgroup holds NW waves: KS key groups of NW / KS waves,
// each group NW / KS / TS consecutive partitions x a team of TS adjacent head
// groups; the team's waves read the same blocks in lockstep.  The key groups'
// states meet in LDS and the first writes the partition's record (or the
// output, for a sequence with one partition).  Grid: x = (sequence * chunks +
// chunk) * (head groups / TS) + block of TS head groups.
// ============================================================================

template <class E, int D, int G, class TU, class A = Engine<E, D, G, TU>>
__global__ __launch_bounds__(TU::NW * kWave) void decode_partition_kernel(DecodeParams p) {
    constexpr int NW = TU::NW;
    constexpr int KS = TU::KS;
    constexpr int NWK = NW / KS;  // waves per key group
    constexpr int NS = A::NS;
    constexpr int DEPTH = TU::DEPTH;
    constexpr int HG = A::HG;
    using Result = typename A::Result;
    constexpr int NF = sizeof(Result) / 4;  // floats of one lane's state
    __shared__ __attribute__((aligned(16))) char sm_eng[NW * (A::kLdsBytes > 0 ? A::kLdsBytes : 16)];
    __shared__ float sm_x[KS > 1 ? (KS - 1) * NWK * NF * kWave : 1];

    const int TS = p.team;
    const int PW = NWK / TS;  // partitions per key group
    const int NG = p.n_kv_heads / A::NH;
    const int NGB = NG / TS;
    const int chunks = (p.n_parts_max + PW - 1) / PW;
    const int hb = blockIdx.x % NGB;
    const int sc = blockIdx.x / NGB;
    const int s = sc / chunks;
    const int w = wave_id_uniform();
    const int kg = w / NWK;  // key group
    const int wl = w - kg * NWK;
    const int pi = wl / TS;
    const int part = (sc - s * chunks) * PW + pi;
    const int hg = hb * TS + (wl - pi * TS);  // head group: KV heads hg*NH .. +NH-1
    const int Hq = p.n_q_heads;
    const int lane = threadIdx.x % kWave;
    char* out_rows = static_cast<char*>(p.out) + ((int64_t)s * Hq + hg * HG) * D * E::kBytes;
    // A length beyond the table is a caller error; clamping keeps every table
    // read inside the row and every partition inside the workspace.
    const int L = min(max(p.context_lens[s], 0), (p.max_blocks << p.block_shift));
    const int P = p.part_tokens;
    const int n_parts = (L + P - 1) / P;
    const bool live = part < n_parts;  // uniform over the wave (not over the workgroup when PW > 1)
    if (L == 0 && part == 0 && kg == 0)  // nothing to attend: zero rows
        for (int i = lane; i < HG * D; i += kWave) E::store(out_rows + i * E::kBytes, 0.f);

    const int nblk = (L + kBlock - 1) / kBlock;
    const int PB = P / kBlock;
    const int HB = (PB + KS - 1) / KS;  // tiles per key group
    const int kb0 = part * PB + kg * HB;
    const int kb1 = live ? min(min(kb0 + HB, part * PB + PB), nblk) : kb0;  // this wave's tiles [kb0, kb1)
    const int tail_rows = L - (nblk - 1) * kBlock;  // valid rows of the last block, 1..16

    const uint32_t row_stride = (uint32_t)p.n_kv_heads * A::RB;
    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)hg * A::NH * A::RB;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)hg * A::NH * A::RB;
    const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks;

    A a;
    a.init(lane, row_stride, sm_eng + w * A::kLdsBytes);
    a.load_q(static_cast<const char*>(p.q) + ((int64_t)s * Hq + hg * HG) * A::RB);
    a.reset();
    bool oks[NS];
    const int ntab = (L + (1 << p.block_shift) - 1) >> p.block_shift;
    // As in the flat schedule: each tile's table entries are read one issue
    // ahead, and every pass issues its loads (past the range's end, of the
    // first rows of block 0, never computed).
    auto fetch = [&](int bi, bool real) {
        TileEnt e = {0, 0};
        if (real) e = tile_entries(table, bi, ntab, p.block_shift);
        return e;
    };
    auto issue = [&](int slot, int bi, TileEnt e, bool real) {
        TileAddr ta = {0, -kDummyRows * (int64_t)row_stride, false};
        if (real) ta = tile_addr_of(e, bi, ntab, p.block_shift, p.num_blocks, row_stride);
        a.template issue<false>(slot, kbase, vbase, ta.lo, ta.hi, -1, kbase, vbase);
        oks[slot] = ta.ok;
    };

    // Block kb0 + k goes through register slot k % NS, DEPTH blocks ahead.
    TileEnt ahead = fetch(kb0, kb0 < kb1);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        issue(d, kb0 + d, ahead, kb0 + d < kb1);
        ahead = fetch(kb0 + d + 1, kb0 + d + 1 < kb1);
    }
    for (int bi = kb0; bi < kb1; bi += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int b = bi + u;
            issue((u + DEPTH) % NS, b + DEPTH, ahead, b + DEPTH < kb1);
            ahead = fetch(b + DEPTH + 1, b + DEPTH + 1 < kb1);
            if (b < kb1) {
                const int valid = !oks[u] ? 0 : (b == nblk - 1 ? tail_rows : kBlock);
                a.process(u, valid, p.scale_log2);
            }
        }
    }
    a.reduce();
    Result r;
    a.take(r);
    if constexpr (KS > 1) {
        // key groups 1.. hand their states to group 0 through LDS, lane by lane
        if (kg > 0) {
            float f[NF];
            __builtin_memcpy(f, &r, sizeof(Result));
            float* x = sm_x + ((kg - 1) * NWK + wl) * NF * kWave;
#pragma unroll
            for (int i = 0; i < NF; ++i) x[i * kWave + lane] = f[i];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int k = 1; k < KS; ++k) {
            const float* x = sm_x + ((k - 1) * NWK + wl) * NF * kWave;
            float f[NF];
#pragma unroll
            for (int i = 0; i < NF; ++i) f[i] = x[i * kWave + lane];
            Result o;
            __builtin_memcpy(&o, f, sizeof(Result));
            A::combine(r, o);
        }
    }
    if (!live) return;
    if (n_parts == 1) {
        a.store_out(r, out_rows);
    } else {  // record [sequence][head group][partition] of [HG][D] acc and [HG][2] (m, l)
        const int64_t rec = ((int64_t)s * NG + hg) * p.n_parts_max + part;
        a.store_partial(r, p.ws_acc + rec * HG * D, p.ws_ml + rec * HG * 2);
    }
}

// Fixed partitions, persistent: the same units of work as
// decode_partition_kernel -- (sequence, partition, block of TS head groups),
// each split between KS key groups that meet in LDS -- and the same bits, but
// a grid of the resident workgroups, each taking a balanced contiguous range
// of units (ordered by sequence, partition, head-group block).  A wave's
// loads run ahead across unit boundaries, so there is no start-up wait per
// partition and no loads issued past a short range's end.  Every wave of a
// workgroup finishes every unit of the range (a key group without tiles in it
// contributes an empty state), so the barriers of the LDS exchange match.
// Requires TS == NW / KS.  LDS: the engine areas, the exchange area and the
// unit prefix over sequences.
template <class E, int D, int G, class TU, class A = Engine<E, D, G, TU>>
__global__ __launch_bounds__(TU::NW * kWave) void decode_partition_persistent_kernel(DecodeParams p) {
    constexpr int NW = TU::NW;
    constexpr int KS = TU::KS;
    constexpr int NWK = NW / KS;  // waves per key group = the team
    constexpr int NS = A::NS;
    constexpr int DEPTH = TU::DEPTH;
    constexpr int HG = A::HG;
    using Result = typename A::Result;
    static_assert(A::kQAhead, "a unit's q rows ride in the slot of its first tile");
    constexpr int SLOT = StageSlot<D, HG>::kFloats;  // one staged state: acc, (m, l), destination
    constexpr int KB = kPartStaged;                  // records a wave stages before writing them
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    char* sm_eng = dyn_lds;
    // exchange slots of key groups 1.. (one per wave), then KB staging slots per wave of group 0
    float* sm_x = reinterpret_cast<float*>(dyn_lds + NW * A::kLdsBytes);
    float* sm_st = sm_x + (KS - 1) * NWK * SLOT;
    int32_t* upre = reinterpret_cast<int32_t*>(sm_st + NWK * KB * SLOT);

    const int S = p.num_seqs;
    const int NG = p.n_kv_heads / A::NH;
    const int NGB = NG / NWK;
    const int Hq = p.n_q_heads;
    const int P = p.part_tokens;
    const int PB = P / kBlock;
    const int HB = (PB + KS - 1) / KS;  // tiles per key group of a partition
    const int max_len = p.max_blocks << p.block_shift;
    auto seq_len = [&](int s) { return min(max(table_entry(p.context_lens, s), 0), max_len); };

    // units of sequence s: n_parts(s) * NGB; upre[s] = units of sequences < s
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        int carry = 0;
        for (int base = 0; base < S; base += kWave) {
            const int i = base + lane;
            // per-lane index: a vector read (seq_len reads a uniform index with a scalar load)
            int v = i < S ? ((min(max(p.context_lens[i], 0), max_len) + P - 1) / P) * NGB : 0;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int y = __shfl_up(v, off, kWave);
                if (lane >= off) v += y;
            }
            if (i < S) upre[i + 1] = carry + v;
            carry += __shfl(v, kWave - 1, kWave);
        }
        if (lane == 0) upre[0] = 0;
    }
    __syncthreads();
    // empty sequences: zero rows (workgroups share them out)
    for (int si = blockIdx.x; si < S; si += gridDim.x)
        if (upre[si + 1] == upre[si]) {
            char* o = static_cast<char*>(p.out) + (int64_t)si * Hq * D * E::kBytes;
            for (int i = threadIdx.x; i < Hq * D; i += blockDim.x) E::store(o + i * E::kBytes, 0.f);
        }
    const int U = upre[S];
    const int u0 = (int)((int64_t)U * blockIdx.x / gridDim.x);
    const int u1 = (int)((int64_t)U * (blockIdx.x + 1) / gridDim.x);
    if (u0 >= u1) return;  // uniform over the workgroup

    const int w = wave_id_uniform();
    const int kg = w / NWK;
    const int tj = w - kg * NWK;
    const int lane = threadIdx.x % kWave;
    const uint32_t row_stride = (uint32_t)p.n_kv_heads * A::RB;

    // Unit cursor: sequence, partition, head-group block, length, and this
    // wave's tiles [kb0, kb1) of the unit (possibly none).
    struct UC {
        int u, s, part, hb, L, kb0, kb1;
    };
    auto set_range = [&](UC& c) {
        const int nblk = (c.L + kBlock - 1) / kBlock;
        c.kb0 = c.part * PB + kg * HB;
        c.kb1 = min(min(c.kb0 + HB, c.part * PB + PB), nblk);
        c.kb1 = max(c.kb1, c.kb0);
    };
    auto uniform = [](UC& c) {
        c.u = __builtin_amdgcn_readfirstlane(c.u);
        c.s = __builtin_amdgcn_readfirstlane(c.s);
        c.part = __builtin_amdgcn_readfirstlane(c.part);
        c.hb = __builtin_amdgcn_readfirstlane(c.hb);
        c.L = __builtin_amdgcn_readfirstlane(c.L);
        c.kb0 = __builtin_amdgcn_readfirstlane(c.kb0);
        c.kb1 = __builtin_amdgcn_readfirstlane(c.kb1);
    };
    auto locate = [&](int u) {
        int lo = 0, hi = S;  // largest s with upre[s] <= u
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (upre[mid] <= u) lo = mid;
            else hi = mid;
        }
        UC c;
        c.u = u;
        c.s = lo;
        c.L = seq_len(lo);
        const int r = u - upre[lo];
        c.part = r / NGB;
        c.hb = r - c.part * NGB;
        set_range(c);
        uniform(c);
        return c;
    };
    auto next_unit = [&](UC& c) {
        ++c.u;
        if (++c.hb == NGB) {
            c.hb = 0;
            ++c.part;
            if (c.part * P >= c.L) {  // past the sequence: the next one with units
                c.part = 0;
                do {
                    ++c.s;
                } while (c.s < S && upre[c.s + 1] == upre[c.s]);
                c.L = c.s < S ? seq_len(c.s) : 0;
            }
        }
        set_range(c);
        uniform(c);
    };

    A a;
    a.init(lane, row_stride, sm_eng + w * A::kLdsBytes);
    a.reset();
    bool oks[NS];

    // Issue cursor: (unit, block) over the wave's tiles of units u0 .. u1-1.
    UC ic = locate(u0);
    int ib = ic.kb0;
    auto skip_empty = [&]() {  // move to the first unit with a tile for this wave, if any
        while (ib >= ic.kb1 && ic.u < u1 - 1) {
            next_unit(ic);
            ib = ic.kb0;
        }
    };
    skip_empty();
    int q_s = -1, q_hb = -1;  // the (sequence, head-group block) whose q rows the last issued tile loaded
    auto issue = [&](int slot) {
        const bool real = ib < ic.kb1;
        TileAddr ta = {0, -kDummyRows * (int64_t)row_stride, false};
        int64_t hoff = 0;
        if (real) {
            const int hg = ic.hb * NWK + tj;
            hoff = (int64_t)hg * A::NH * A::RB;
            if (ic.s != q_s || ic.hb != q_hb) {
                q_s = ic.s;
                q_hb = ic.hb;
                a.load_q_slot(slot, static_cast<const char*>(p.q) + ((int64_t)ic.s * Hq + hg * HG) * A::RB);
            }
            const int ntab = (ic.L + (1 << p.block_shift) - 1) >> p.block_shift;
            ta = tile_addr(p.block_tables + (int64_t)ic.s * p.max_blocks, ib, ntab, p.block_shift, p.num_blocks,
                           row_stride);
        }
        const char* kb = static_cast<const char*>(p.k_cache) + hoff;
        const char* vb = static_cast<const char*>(p.v_cache) + hoff;
        a.template issue<false>(slot, kb, vb, ta.lo, ta.hi, -1, kb, vb);
        oks[slot] = ta.ok;
        if (real) {
            ++ib;
            skip_empty();
        }
    };

    // Processing cursor and the unit being accumulated.
    UC pc = locate(u0);
    int pb = pc.kb0;
    int cu = u0;  // the next unit to finish
    int cq_s = -1, cq_hb = -1;

    // Finished records wait in LDS (KB per wave of key group 0) and are written
    // together (see write_staged).
    int nst = 0;
    const float* const xs_own = sm_x + ((kg > 0 ? kg - 1 : 0) * NWK + tj) * SLOT;
    float* const st_own = sm_st + tj * KB * SLOT;
    auto flush = [&]() {
        write_staged<E, D, HG>(st_own, nst, p);
        nst = 0;
    };

    // Finish unit cu: combine the key groups' states and stage its record.
    auto finish = [&]() {
        a.reduce();
        Result r;
        a.take(r);
        if constexpr (KS > 1) {
            if (kg > 0) a.stage(r, const_cast<float*>(xs_own));
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int k = 1; k < KS; ++k) {
                    Result o;
                    a.unstage(sm_x + ((k - 1) * NWK + tj) * SLOT, o);
                    A::combine(r, o);
                }
            }
            __syncthreads();  // the exchange slots are free again
        }
        if (kg == 0) {
            // pc is still at unit cu here (it moves on after finish)
            const int hg = pc.hb * NWK + tj;
            const int n_parts = (pc.L + P - 1) / P;
            float* sl = st_own + nst * SLOT;
            a.stage(r, sl);
            const int64_t dst = n_parts == 1 ? (int64_t)pc.s * Hq + hg * HG
                                             : ((int64_t)pc.s * NG + hg) * p.n_parts_max + pc.part;
            stage_header(sl, SLOT, n_parts == 1, dst);
            if (++nst == KB) flush();
        }
        a.reset();
        ++cu;
        if (cu < u1) {
            next_unit(pc);
            pb = pc.kb0;
        }
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d);
    // Each pass processes one tile of this wave (after finishing the units
    // that precede it), or, once the tiles are done, finishes the rest.
    bool more = true;
    while (more) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            issue((u + DEPTH) % NS);
            // units with no tile left for this wave are finished first
            while (cu < u1 && pb >= pc.kb1) finish();
            if (cu < u1) {
                if (pc.s != cq_s || pc.hb != cq_hb) {
                    cq_s = pc.s;
                    cq_hb = pc.hb;
                    a.take_q(u);
                }
                const int nblk = (pc.L + kBlock - 1) / kBlock;
                const int valid = !oks[u] ? 0 : (pb == nblk - 1 ? pc.L - (nblk - 1) * kBlock : kBlock);
                a.process(u, valid, p.scale_log2);
                ++pb;
            } else {
                more = false;
            }
        }
    }
    if (kg == 0 && nst > 0) flush();
}

// Fixed partitions: one 512-thread workgroup per (sequence, query head) whose
// sequence has >= 2 partitions.  A long sequence has hundreds of records, so
// the workgroup reads RS records side by side (thread t owns float4 column
// t % VPR of record slot t / VPR), UNROLL deep (128 records of D = 128 in
// flight), and the slots' partial sums meet in LDS.
constexpr int kMergeThreads = 512;

template <class E, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeParams p) {
    constexpr int NT = kMergeThreads;
    constexpr int NWV = NT / kWave;
    constexpr int VPR = D / 4;    // float4 columns of a record row
    constexpr int RS = NT / VPR;  // record slots
    constexpr int UNROLL = 8;
    __shared__ float sm_max[NWV], sm_den[NWV];
    __shared__ __attribute__((aligned(16))) float4 sm_num[RS][VPR];

    const int pair = blockIdx.x;
    const int s = pair / p.n_q_heads;
    const int h = pair % p.n_q_heads;
    const int L = min(max(p.context_lens[s], 0), (p.max_blocks << p.block_shift));
    const int n = (L + p.part_tokens - 1) / p.part_tokens;
    if (n < 2) return;  // uniform over the workgroup
    const int HG = p.n_q_heads / p.n_kv_heads * p.heads_per_wave;  // query heads per record
    const int NG = p.n_kv_heads / p.heads_per_wave;
    const int hg = h / HG;
    // record x of this head: row (first + x * HG) of acc ([.][D]) and ml ([.][2])
    const int64_t first = ((int64_t)s * NG + hg) * p.n_parts_max * HG + h % HG;
    const float* ml = p.ws_ml;
    const float* acc = p.ws_acc;
    const int tid = threadIdx.x;
    const int wv = tid / kWave;

    float M = -INFINITY;
    for (int x = tid; x < n; x += NT) M = fmaxf(M, ml[(first + (int64_t)x * HG) * 2]);
    M = wave_max(M);
    if (tid % kWave == 0) sm_max[wv] = M;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NWV; ++i) M = fmaxf(M, sm_max[i]);

    float den = 0.f;
    for (int x = tid; x < n; x += NT) {
        const int64_t r = first + (int64_t)x * HG;
        den += __builtin_amdgcn_exp2f(ml[r * 2] - M) * ml[r * 2 + 1];
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) den += shfl_xor(den, m);
    if (tid % kWave == 0) sm_den[wv] = den;

    const int c = tid % VPR;
    const int slot = tid / VPR;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int x0 = slot; x0 < n; x0 += RS * UNROLL) {
        float f[UNROLL];
        float4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int x = x0 + u * RS;
            const bool ok = x < n;
            const int64_t r = first + (int64_t)(ok ? x : 0) * HG;
            f[u] = ok ? __builtin_amdgcn_exp2f(ml[r * 2] - M) : 0.f;
            v[u] = *reinterpret_cast<const float4*>(acc + r * D + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            num.x = __builtin_fmaf(f[u], v[u].x, num.x);
            num.y = __builtin_fmaf(f[u], v[u].y, num.y);
            num.z = __builtin_fmaf(f[u], v[u].z, num.z);
            num.w = __builtin_fmaf(f[u], v[u].w, num.w);
        }
    }
    sm_num[slot][c] = num;
    __syncthreads();
    if (tid < VPR) {
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < NWV; ++i) tot += sm_den[i];
        const float inv = 1.f / tot;
        float4 o = sm_num[0][tid];
#pragma unroll
        for (int r = 1; r < RS; ++r) {
            const float4 y = sm_num[r][tid];
            o.x += y.x;
            o.y += y.y;
            o.z += y.z;
            o.w += y.w;
        }
        char* out_row = static_cast<char*>(p.out) + ((int64_t)pair * D + 4 * tid) * E::kBytes;
        E::store(out_row, o.x * inv);
        E::store(out_row + E::kBytes, o.y * inv);
        E::store(out_row + 2 * E::kBytes, o.z * inv);
        E::store(out_row + 3 * E::kBytes, o.w * inv);
    }
}

// ============================================================================
// Dispatch
// ============================================================================

// Launch shape per element type, head_dim and group size (chosen by measured
// sweeps on MI355X).  16-bit caches with G >= 4 use the matrix-core engine:
// under the flat schedule 8 waves per workgroup with two tiles in flight at
// G = 4, one wave with one tile in flight at G = 8 (its larger score tile
// leaves fewer registers for prefetch); under fixed partitions one wave per
// workgroup with two tiles in flight, so that a wave streams its partition
// alone and no workgroup waits on its slowest wave.  Other 16-bit caches use
// the vector engine streaming two adjacent KV heads per wave (16 lanes per head
// row, so one load instruction reads two tokens x 512 contiguous bytes at
// D = 128); fp32 caches one head per wave.  NH1 is the one-head shape used
// when the KV head count is odd (it must match `type` in everything but NH).
// Share of a workgroup's tiles taken by its first team (waves 0-3) when its
// 8 waves form two teams of 4 (see decode_flat_kernel).  Measured on the
// GQA-8B, copied-prefix and long-context layers: 50 % (equal shares) 5.85,
// 5.89, 6.39 TB/s; 58 %: 5.95, 6.01, 6.53; 62 %: 6.02, 6.09, 6.65; 66 %: 5.97,
// 6.10, 6.64; 70 %: 5.90, 6.04, 6.48 (one team of 8 waves: 5.85, 5.86,
// 6.50).
constexpr int kSplitPct = 62;
// Share of two consecutive workgroups' tiles taken by the first, which runs on
// an even XCD (see decode_flat_kernel).  Matrix-core engine, GQA-8B layer: 50 %
// 6.03 TB/s, 52 %: 6.11, 54 %: 6.04, 56 %: 5.95; vector engine, Llama-2-7B
// layer (four runs each, back to back): 53 % 6.37, 54 %: 6.42, 55 %: 6.39,
// 56 %: 6.34, 57 %: 6.28.
constexpr int kXcdPctMfma = 52;
constexpr int kXcdPctValu = 54;

template <class E, int D, int G>
struct DefaultTune {
    static constexpr bool kMfma = E::kBytes == 2 && G >= 4;
    static constexpr int kCH = D * E::kBytes / 16;
    static constexpr int kR = kCH < 16 ? kCH : 16;
    static constexpr int kNH = E::kBytes == 2 && !kMfma ? 2 : 1;
    // matrix-core engine: 8-wave workgroups in two teams of 4 (each team
    // streams 4 KV heads of the same blocks together), the first taking
    // kSplitPct of the pair's tiles
    using mfma_flat = Tune<8, 8, 1, true, true, 1, 0, 4>;
    // fp32 with G >= 4 spreads a head row over more lanes: fewer accumulators per lane
    static constexpr int kRf = E::kBytes == 4 && G >= 4 ? kR : 8;
    // 16-bit, two KV heads a wave: one 4-wave workgroup per CU (one wave per
    // SIMD) streams 2-3 % faster than the two waves per SIMD that fit
    using valu = typename std::conditional<kNH == 2, Tune<4, kR, 1, true, false, 2, 1>, Tune<4, kRf, 1, true, false, 1>>::type;
    using type = typename std::conditional<kMfma, mfma_flat, valu>::type;
    // fixed partitions: a partition's tiles split between two key groups, each
    // a team of four KV heads (the tail of a grid of equal partitions is half as long)
    using parts = typename std::conditional<kMfma, Tune<8, 8, 1, true, true, 1, 0, 4, 2>, valu>::type;
    using NH1 = Tune<4, kMfma ? 8 : kRf, 1, true, kMfma, 1>;
};

template <class E, int D, int G>
static int heads_per_wave_t(int n_kv_heads) {
    constexpr int nh = DefaultTune<E, D, G>::type::NH;
    return n_kv_heads % nh == 0 ? nh : 1;
}

// Team size of the flat schedule's launch for this shape (the merge pass needs it).
template <class E, int D, int G>
static int flat_team_t(int n_kv_heads) {
    using TU = typename DefaultTune<E, D, G>::type;
    using TU1 = typename DefaultTune<E, D, G>::NH1;
    return heads_per_wave_t<E, D, G>(n_kv_heads) == TU::NH ? team_size<TU>(n_kv_heads / TU::NH)
                                                            : team_size<TU1>(n_kv_heads);
}

// Fixed partitions, one workgroup per (partition, team) (p.team set).
template <class E, int D, int G, class TU, class A = Engine<E, D, G, TU>>
hipError_t launch_parts_fallback(const DecodeParams& p, hipStream_t stream) {
    const int ng = p.n_kv_heads / A::NH;
    const int pw = TU::NW / TU::KS / p.team;  // partitions per key group
    const int64_t chunks = (p.n_parts_max + pw - 1) / pw;
    const int64_t wgs = chunks * p.num_seqs * (ng / p.team);
    if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_partition_kernel<E, D, G, TU, A>), dim3((unsigned)wgs), dim3(TU::NW * kWave), 0,
                       stream, p);
    return hipGetLastError();
}

template <class E, int D, int G, class TU, class A = Engine<E, D, G, TU>>
hipError_t launch_parts_persistent(const DecodeParams& pin, hipStream_t stream);

// Largest LDS the persistent partition kernel asks for (beyond it, the batch
// has too many sequences for the unit prefix and the one-launch-per-partition
// kernel runs instead; both give the same bits).
constexpr size_t kMaxPersistentLds = 160 * 1024;

template <class E, int D, int G, class TU, class A = Engine<E, D, G, TU>>
hipError_t launch_parts_tuned(const DecodeParams& pin, hipStream_t stream) {
    DecodeParams p = pin;
    p.heads_per_wave = A::NH;
    const int ng = p.n_kv_heads / A::NH;
    p.team = team_size<TU>(ng);
    // The persistent kernel when the team fills a key group.
    if constexpr (TU::KS > 1)
        if (p.team == TU::NW / TU::KS) return launch_parts_persistent<E, D, G, TU, A>(p, stream);
    return launch_parts_fallback<E, D, G, TU, A>(p, stream);
}

// One workgroup per resident slot on the device (at most one per unit of work).
template <class E, int D, int G, class TU, class A>
hipError_t launch_parts_persistent(const DecodeParams& p, hipStream_t stream) {
    auto kern = decode_partition_persistent_kernel<E, D, G, TU, A>;
    constexpr size_t slot = (size_t)StageSlot<D, A::HG>::kFloats * 4;
    const size_t lds = (size_t)TU::NW * A::kLdsBytes + (size_t)(TU::KS - 1) * (TU::NW / TU::KS) * slot +
                       (size_t)(TU::NW / TU::KS) * kPartStaged * slot + (size_t)(p.num_seqs + 1) * sizeof(int32_t);
    if (lds > kMaxPersistentLds) return launch_parts_fallback<E, D, G, TU, A>(p, stream);
    static thread_local int cached_dev = -1, cached_per_cu = 0, cached_cus = 0;
    static thread_local size_t cached_lds = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev != cached_dev || lds != cached_lds) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, TU::NW * kWave, lds);
        if (e != hipSuccess) return e;
        cached_dev = dev;
        cached_lds = lds;
        cached_cus = cus;
        cached_per_cu = per_cu < 1 ? 1 : per_cu;
    }
    const int64_t units = (int64_t)p.num_seqs * p.n_parts_max * (p.n_kv_heads / A::NH / p.team);
    int64_t wgs = (int64_t)cached_cus * cached_per_cu;
    if (wgs > units) wgs = units;
    if (wgs < 1) wgs = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(TU::NW * kWave), lds, stream, p);
    return hipGetLastError();
}

// Workgroups of the flat kernel resident on the whole device, capped so the
// grid's waves never exceed kMaxFlatWorkers.
template <class E, int D, int G, class TU, class A = Engine<E, D, G, TU>>
hipError_t launch_flat_tuned(const DecodeParams& pin, hipStream_t stream) {
    DecodeParams p = pin;
    p.heads_per_wave = A::NH;
    p.team = team_size<TU>(p.n_kv_heads / A::NH);
    // the first of two teams of a workgroup takes this share of their tiles,
    // a workgroup on an even XCD this share of a pair's
    p.split_pct = TU::NW / p.team == 2 ? kSplitPct : 50;
    p.xcd_pct = TU::MFMA ? kXcdPctMfma : kXcdPctValu;
    // The grid is sized from the kernel without the fused append, and the fused
    // kernel gets the same grid: the tiles are then dealt alike and both give
    // the same bits.  (Its waves do not wait on one another, so a grid larger
    // than what is resident would only run in turns.)
    auto kern_plain = decode_flat_kernel<E, D, G, TU, false, A>;
    auto kern = p.positions != nullptr ? decode_flat_kernel<E, D, G, TU, true, A> : kern_plain;
    const size_t lds = (size_t)TU::NW * A::kLdsBytes + (size_t)(2 * p.num_seqs + 1) * sizeof(int32_t);
    static thread_local int cached_dev = -1, cached_per_cu = 0, cached_cus = 0;
    static thread_local size_t cached_lds = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev != cached_dev || lds != cached_lds) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern_plain, TU::NW * kWave, lds);
        if (e != hipSuccess) return e;
        cached_dev = dev;
        cached_lds = lds;
        cached_cus = cus;
        cached_per_cu = per_cu < 1 ? 1 : per_cu;
        if (TU::CAP > 0 && cached_per_cu > TU::CAP) cached_per_cu = TU::CAP;
    }
    int wgs = cached_cus * cached_per_cu;
    if (wgs * TU::NW > kMaxFlatWorkers) wgs = kMaxFlatWorkers / TU::NW;
    hipLaunchKernelGGL(kern, dim3(wgs), dim3(TU::NW * kWave), lds, stream, p);
    return hipGetLastError();
}

template <class E, int D, int G>
static hipError_t launch_g(const DecodeParams& p, bool flat, hipStream_t stream) {
    using TU = typename DefaultTune<E, D, G>::type;
    using TP = typename DefaultTune<E, D, G>::parts;
    using TU1 = typename DefaultTune<E, D, G>::NH1;
    static_assert(TU::NH == TP::NH, "both schedules must group KV heads alike (the merge pass assumes it)");
    if (heads_per_wave_t<E, D, G>(p.n_kv_heads) == TU::NH)
        return flat ? launch_flat_tuned<E, D, G, TU>(p, stream) : launch_parts_tuned<E, D, G, TP>(p, stream);
    return flat ? launch_flat_tuned<E, D, G, TU1>(p, stream) : launch_parts_tuned<E, D, G, TU1>(p, stream);
}

template <class E, int D>
static hipError_t launch_d(const DecodeParams& p, int group, bool flat, hipStream_t stream) {
    switch (group) {
        case 1: return launch_g<E, D, 1>(p, flat, stream);
        case 2: return launch_g<E, D, 2>(p, flat, stream);
        case 4: return launch_g<E, D, 4>(p, flat, stream);
        case 8: return launch_g<E, D, 8>(p, flat, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
static hipError_t launch_e(const DecodeParams& p, int head_dim, int group, bool flat, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_d<E, 64>(p, group, flat, stream);
        case 128: return launch_d<E, 128>(p, group, flat, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E, int D>
static int heads_per_wave_d(int group, int n_kv_heads) {
    switch (group) {
        case 1: return heads_per_wave_t<E, D, 1>(n_kv_heads);
        case 2: return heads_per_wave_t<E, D, 2>(n_kv_heads);
        case 4: return heads_per_wave_t<E, D, 4>(n_kv_heads);
        case 8: return heads_per_wave_t<E, D, 8>(n_kv_heads);
        default: return 1;
    }
}

template <class E>
static int heads_per_wave_e(int head_dim, int group, int n_kv_heads) {
    return head_dim == 64 ? heads_per_wave_d<E, 64>(group, n_kv_heads)
                          : heads_per_wave_d<E, 128>(group, n_kv_heads);
}

template <class E, int D>
static int flat_team_d(int group, int n_kv_heads) {
    switch (group) {
        case 1: return flat_team_t<E, D, 1>(n_kv_heads);
        case 2: return flat_team_t<E, D, 2>(n_kv_heads);
        case 4: return flat_team_t<E, D, 4>(n_kv_heads);
        case 8: return flat_team_t<E, D, 8>(n_kv_heads);
        default: return 1;
    }
}

template <class E>
static int flat_team_e(int head_dim, int group, int n_kv_heads) {
    return head_dim == 64 ? flat_team_d<E, 64>(group, n_kv_heads) : flat_team_d<E, 128>(group, n_kv_heads);
}

int decode_heads_per_wave(int dtype, int head_dim, int group, int n_kv_heads) {
    switch (dtype) {
        case 0: return heads_per_wave_e<F32>(head_dim, group, n_kv_heads);
        case 1: return heads_per_wave_e<F16>(head_dim, group, n_kv_heads);
        case 2: return heads_per_wave_e<BF16>(head_dim, group, n_kv_heads);
        default: return 1;
    }
}

bool decode_supported(int dtype, int head_dim, int group) {
    return dtype >= 0 && dtype <= 2 && (head_dim == 64 || head_dim == 128) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_partitions(const DecodeParams& p, int dtype, int head_dim, int group,
                                    hipStream_t stream) {
    const bool flat = p.part_tokens == 0;
    switch (dtype) {
        case 0: return launch_e<F32>(p, head_dim, group, flat, stream);
        case 1: return launch_e<F16>(p, head_dim, group, flat, stream);
        case 2: return launch_e<BF16>(p, head_dim, group, flat, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
static hipError_t launch_merge_e(const DecodeParams& pin, int head_dim, int group, hipStream_t stream) {
    DecodeParams p = pin;
    p.heads_per_wave = heads_per_wave_e<E>(head_dim, group, p.n_kv_heads);
    p.team = flat_team_e<E>(head_dim, group, p.n_kv_heads);
    const int pairs = p.num_seqs * p.n_q_heads;
    const dim3 grid_flat((pairs + 3) / 4);  // one wave per pair
    const dim3 grid_parts(pairs);           // one workgroup per pair
    const bool flat = p.part_tokens == 0;
    switch (head_dim) {
        case 64:
            if (flat) hipLaunchKernelGGL((decode_flat_merge_kernel<E, 64>), grid_flat, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((decode_merge_kernel<E, 64>), grid_parts, dim3(kMergeThreads), 0, stream, p);
            break;
        case 128:
            if (flat) hipLaunchKernelGGL((decode_flat_merge_kernel<E, 128>), grid_flat, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((decode_merge_kernel<E, 128>), grid_parts, dim3(kMergeThreads), 0, stream, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& p, int dtype, int head_dim, int group, hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_merge_e<F32>(p, head_dim, group, stream);
        case 1: return launch_merge_e<F16>(p, head_dim, group, stream);
        case 2: return launch_merge_e<BF16>(p, head_dim, group, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
