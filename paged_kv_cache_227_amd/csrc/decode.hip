// decode.hip -- paged decode attention on gfx950: split-K partition pass and
// log-sum-exp merge.
//
// What is computed: for sequence s, query head h, KV head g = h / G
// (G = n_q_heads / n_kv_heads) and L = context_lens[s],
//     out[s][h] = sum_{i<L} softmax_i(scale * <q[s][h], K_i>) V_i
// where K_i, V_i are row (i mod B) of physical block block_table[s][i / B]
// ("How a serving engine actually works", paperfordummies.in, "The one
// formula"; the attention maths is unchanged by paging -- henryhe.ai,
// "What's deliberately still missing").
//
// Partition pass (one workgroup per (partition j, KV head g, sequence s)):
//   * a partition is P consecutive tokens (P / 16 whole blocks); its blocks
//     are dealt round-robin to the workgroup's NW waves;
//   * a wave streams one 16-token block at a time: the K tile and the V tile
//     of head g (16 rows of head_dim elements, rows n_kv_heads * head_dim
//     elements apart) with 16-byte loads, R = 8 lanes per row so that one
//     load instruction reads 8 rows x 128 contiguous bytes; the next block's
//     tiles are loaded while the current one is computed;
//   * the G query heads that share head g reuse every K/V register tile, so
//     each K/V byte leaves HBM once per step;
//   * QK: packed 16-bit dot products with fp32 accumulation (v_dot2), summed
//     over the 8 lanes of a row with DPP; scores are kept in base-2 units
//     (scale * log2 e folded in) so the softmax uses v_exp_f32 directly;
//   * online softmax per row group of lanes: running max m, sum l and the
//     unnormalised accumulator acc; acc is rescaled only when some lane's max
//     grows; rows past L (last block only) are masked by select, values too,
//     so whatever those slots hold (NaN included) never reaches the output;
//   * epilogue: the row groups of a wave, then the NW waves (through LDS),
//     are combined by the log-sum-exp rule; a sequence whose context fits one
//     partition gets its normalised output written here (rounded to the
//     cache dtype), otherwise (m, l, acc) go to the workspace.
// Merge pass (one wave per (s, h), sequences with >= 2 partitions only):
//     M = max_j m_j,  out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j.
//
// Everything is bound by HBM bandwidth: each (token, KV head) costs
// 2 * head_dim * element bytes of reads and 4 * head_dim * G flops.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kLanesPerRow = 8;
constexpr int kWavesPerGroup = 4;

template <class E, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_partition_kernel(DecodeParams p) {
    constexpr int VEC = E::kPerVec;       // elements per 16-byte vector
    constexpr int RB = D * E::kBytes;     // bytes per (token, head) row
    constexpr int CH = RB / 16;           // 16-byte chunks per row
    constexpr int R = kLanesPerRow;       // lanes sharing one row
    constexpr int CPL = CH / R;           // chunks per lane per row
    constexpr int RPS = kWave / R;        // rows covered by one load instruction
    constexpr int J = kBlock / RPS;       // rows per lane per block
    constexpr int EPL = CPL * VEC;        // elements per lane per row
    static_assert(CH % R == 0 && kBlock % RPS == 0, "row / lane mapping");

    const int part = blockIdx.x;
    const int kvh = blockIdx.y;
    const int s = blockIdx.z;
    const int Hq = p.n_q_heads;
    const int h0 = kvh * G;
    // A length beyond the table is a caller error; clamping keeps every table
    // read inside the row and every partition inside the workspace.
    const int L = min(max(p.context_lens[s], 0), p.max_blocks * kBlock);
    const int P = p.part_tokens;
    const int n_parts = (L + P - 1) / P;

    if (part >= n_parts) {
        if (L == 0 && part == 0) {  // nothing to attend: a zero row
            for (int i = threadIdx.x; i < G * D; i += blockDim.x)
                E::store(static_cast<char*>(p.out) +
                             (((int64_t)s * Hq + h0 + i / D) * D + i % D) * E::kBytes,
                         0.f);
        }
        return;
    }

    const int lane = threadIdx.x % kWave;
    const int w = wave_id_uniform();
    const int rg = lane / R;  // row group
    const int c = lane % R;   // chunk column

    const int nblk = (L + kBlock - 1) / kBlock;
    const int PB = P / kBlock;
    const int b_begin = part * PB;
    const int b_end = min(b_begin + PB, nblk);
    const int tail_rows = L - (nblk - 1) * kBlock;  // valid rows of the last block, 1..16

    const uint32_t row_stride = (uint32_t)p.n_kv_heads * RB;  // bytes between token rows
    const int64_t blk_bytes = (int64_t)row_stride * kBlock;
    const char* kbase = static_cast<const char*>(p.k_cache) + (int64_t)kvh * RB;
    const char* vbase = static_cast<const char*>(p.v_cache) + (int64_t)kvh * RB;
    const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks;

    uint32_t lane_off[J][CPL];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int k = 0; k < CPL; ++k) lane_off[j][k] = (j * RPS + rg) * row_stride + (c + k * R) * 16;

    // Query vectors of the G heads, the same chunks as this lane's K chunks.
    Vec16 qv[G][CPL];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
            qv[gi][k] = load16(static_cast<const char*>(p.q) +
                               (((int64_t)s * Hq + h0 + gi) * D) * E::kBytes + (c + k * R) * 16);

    float acc[G][EPL];
    float m[G], l[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        m[gi] = -INFINITY;
        l[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[gi][e] = 0.f;
    }

    Vec16 kb[2][J][CPL], vb[2][J][CPL];

    auto issue = [&](int buf, int bi) {
        int pb = __builtin_amdgcn_readfirstlane(table[bi]);
        if (pb < 0 || pb >= p.num_blocks) pb = -1;
        const int64_t boff = pb < 0 ? 0 : (int64_t)pb * blk_bytes;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                kb[buf][j][k] = load16(kbase + boff + lane_off[j][k]);
                vb[buf][j][k] = load16(vbase + boff + lane_off[j][k]);
            }
        return pb;
    };

    auto process = [&](int buf, int bi, int pb) {
        // rows of this block that belong to the sequence
        const int valid = pb < 0 ? 0 : (bi == nblk - 1 ? tail_rows : kBlock);
        float sc[G][J];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                float d = 0.f;
#pragma unroll
                for (int k = 0; k < CPL; ++k) d = E::dot(qv[gi][k], kb[buf][j][k], d);
                sc[gi][j] = group_sum<R>(d) * p.scale_log2;
            }
        float vf[J][EPL];
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int k = 0; k < CPL; ++k) E::expand(vb[buf][j][k], &vf[j][k * VEC]);
        if (valid < kBlock) {  // wave-uniform: only the last block, or a skipped one
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const bool ok = j * RPS + rg < valid;
#pragma unroll
                for (int gi = 0; gi < G; ++gi) sc[gi][j] = ok ? sc[gi][j] : -INFINITY;
#pragma unroll
                for (int e = 0; e < EPL; ++e) vf[j][e] = ok ? vf[j][e] : 0.f;
            }
        }
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
                const float pj = __builtin_amdgcn_exp2f(sc[gi][j] - ms);
                l[gi] += pj;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[gi][e] = __builtin_fmaf(pj, vf[j][e], acc[gi][e]);
            }
        }
    };

    // Software pipeline: tiles of block i + NW load while block i computes.
    int bi = b_begin + w;
    int pb0 = 0, pb1 = 0;
    if (bi < b_end) pb0 = issue(0, bi);
    for (; bi < b_end; bi += 2 * NW) {
        const int b1 = bi + NW;
        if (b1 < b_end) pb1 = issue(1, b1);
        process(0, bi, pb0);
        const int b2 = b1 + NW;
        if (b2 < b_end) pb0 = issue(0, b2);
        if (b1 < b_end) process(1, b1, pb1);
    }

    // Combine the row groups of this wave (lanes c, c+8, ..., c+56).
    float lw[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        float M = m[gi];
#pragma unroll
        for (int x = R; x < kWave; x <<= 1) M = fmaxf(M, shfl_xor(M, x));
        const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[gi] - M);
        float lsum = l[gi] * f;
#pragma unroll
        for (int x = R; x < kWave; x <<= 1) lsum += shfl_xor(lsum, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float a = acc[gi][e] * f;
#pragma unroll
            for (int x = R; x < kWave; x <<= 1) a += shfl_xor(a, x);
            acc[gi][e] = a;
        }
        m[gi] = M;
        lw[gi] = lsum;
    }

    // Combine the waves through LDS.
    __shared__ float sm_acc[NW][G][D];
    __shared__ float sm_m[NW][G];
    __shared__ float sm_l[NW][G];
    if (rg == 0) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
#pragma unroll
            for (int k = 0; k < CPL; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) sm_acc[w][gi][(c + k * R) * VEC + e] = acc[gi][k * VEC + e];
            if (c == 0) {
                sm_m[w][gi] = m[gi];
                sm_l[w][gi] = lw[gi];
            }
        }
    }
    __syncthreads();

    const bool single = n_parts == 1;
    for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
        const int gi = i / D;
        const int d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < NW; ++x) M = fmaxf(M, sm_m[x][gi]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int x = 0; x < NW; ++x) {
            const float f = sm_m[x][gi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[x][gi] - M);
            num = __builtin_fmaf(f, sm_acc[x][gi][d], num);
            den = __builtin_fmaf(f, sm_l[x][gi], den);
        }
        const int64_t row = (int64_t)s * Hq + h0 + gi;
        if (single) {
            E::store(static_cast<char*>(p.out) + (row * D + d) * E::kBytes, num / den);
        } else {
            const int64_t slot = row * p.n_parts_max + part;
            p.ws_acc[slot * D + d] = num;
            if (d == 0) {
                p.ws_ml[slot * 2] = M;
                p.ws_ml[slot * 2 + 1] = den;
            }
        }
    }
}

// One wave per (sequence, query head); only sequences split into >= 2 partitions.
template <class E, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
    constexpr int PER = (D + kWave - 1) / kWave;
    const int lane = threadIdx.x % kWave;
    const int pair = blockIdx.x * (blockDim.x / kWave) + wave_id_uniform();
    if (pair >= p.num_seqs * p.n_q_heads) return;
    const int s = pair / p.n_q_heads;
    const int L = min(max(p.context_lens[s], 0), p.max_blocks * kBlock);
    const int n = (L + p.part_tokens - 1) / p.part_tokens;
    if (n < 2) return;
    const int64_t base = (int64_t)pair * p.n_parts_max;
    const float* ml = p.ws_ml + base * 2;
    const float* acc = p.ws_acc + base * D;

    float M = -INFINITY;
    for (int j = lane; j < n; j += kWave) M = fmaxf(M, ml[2 * j]);
    M = wave_max(M);

    float num[PER], den = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] = 0.f;
    for (int j = 0; j < n; ++j) {
        const float f = __builtin_amdgcn_exp2f(ml[2 * j] - M);
        den = __builtin_fmaf(f, ml[2 * j + 1], den);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int d = lane + k * kWave;
            if (d < D) num[k] = __builtin_fmaf(f, acc[(int64_t)j * D + d], num[k]);
        }
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = lane + k * kWave;
        if (d < D)
            E::store(static_cast<char*>(p.out) + ((int64_t)pair * D + d) * E::kBytes, num[k] * inv);
    }
}

// ---- dispatch ------------------------------------------------------------------

template <class E, int D, int G>
static hipError_t launch_parts_t(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid(p.n_parts_max, p.n_kv_heads, p.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<E, D, G, kWavesPerGroup>), grid,
                       dim3(kWavesPerGroup * kWave), 0, stream, p);
    return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_parts_g(const DecodeParams& p, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_parts_t<E, D, 1>(p, stream);
        case 2: return launch_parts_t<E, D, 2>(p, stream);
        case 4: return launch_parts_t<E, D, 4>(p, stream);
        case 8: return launch_parts_t<E, D, 8>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
static hipError_t launch_parts_d(const DecodeParams& p, int head_dim, int group, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_parts_g<E, 64>(p, group, stream);
        case 128: return launch_parts_g<E, 128>(p, group, stream);
        default: return hipErrorInvalidValue;
    }
}

bool decode_supported(int dtype, int head_dim, int group) {
    return dtype >= 0 && dtype <= 2 && (head_dim == 64 || head_dim == 128) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_partitions(const DecodeParams& p, int dtype, int head_dim, int group,
                                    hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_parts_d<F32>(p, head_dim, group, stream);
        case 1: return launch_parts_d<F16>(p, head_dim, group, stream);
        case 2: return launch_parts_d<BF16>(p, head_dim, group, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
static hipError_t launch_merge_d(const DecodeParams& p, int head_dim, hipStream_t stream) {
    const int pairs = p.num_seqs * p.n_q_heads;
    const dim3 grid((pairs + 3) / 4);
    switch (head_dim) {
        case 64: hipLaunchKernelGGL((decode_merge_kernel<E, 64>), grid, dim3(256), 0, stream, p); break;
        case 128: hipLaunchKernelGGL((decode_merge_kernel<E, 128>), grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& p, int dtype, int head_dim, hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_merge_d<F32>(p, head_dim, stream);
        case 1: return launch_merge_d<F16>(p, head_dim, stream);
        case 2: return launch_merge_d<BF16>(p, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
