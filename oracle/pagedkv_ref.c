/*
 * pagedkv_ref.c -- CPU oracle for the paged KV cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  The product
 * (the HIP library under paged_kv_cache_227_amd/csrc) never calls it, and
 * the two share no code, headers, tables or helpers.
 *
 * It is plain, slow and meant to be checked by eye:
 *   - every stored element is decoded to double from its bit-level format
 *     definition (IEEE-754 binary32 / binary16, bfloat16);
 *   - attention is the textbook two-pass softmax, accumulated in double;
 *   - K/V rows are located with the address translation of
 *     "How a serving engine actually works" (paperfordummies.in), section
 *     "The one formula":  slot = block_table[seq][i / B] * B + (i mod B);
 *   - per-layer caches are laid out [num_blocks][B][n_kv_heads][head_dim],
 *     indexed by physical block ("Paged-KV + Continuous Batching From
 *     Scratch", henryhe.ai, section 1; snowch.github.io ch08, "The build").
 *
 * Readings of points the pages leave open (query head h uses KV head
 * h / (Hq/Hkv); no causal mask; context_len 0 gives zeros; rows past the
 * context length are never read) are stated beside the code that takes them.
 *
 * Every function is pinned by tests against values the pages print, closed
 * forms, invariants and library routines (torch / numpy); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_F32 0
#define REF_F16 1
#define REF_BF16 2

#define REF_OK 0
#define REF_EINVAL 1

/* ------------------------------------------------------------------------ */
/* Storage formats, decoded and encoded from their definitions.              */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double ref_f16_bits_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal: m * 2^(1-15-10) */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is, by definition, the upper 16 bits of a binary32. */
double ref_bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to a binary format with `mant` fraction bits and `ebits`
 * exponent bits, round-to-nearest-even, directly from the double (no
 * intermediate binary32, so no double rounding).  Overflow gives infinity;
 * NaN gives the quiet NaN with only the top fraction bit set.
 */
static uint16_t ref_encode_small_float(double x, int mant, int ebits) {
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const int emax = bias;
    const uint16_t sign = signbit(x) ? (uint16_t)(1u << (mant + ebits)) : 0;
    const uint16_t exp_all = (uint16_t)(((1u << ebits) - 1) << mant);
    if (isnan(x)) return (uint16_t)(sign | exp_all | (1u << (mant - 1)));
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | exp_all);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1): a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < emin) E = emin; /* subnormal range shares the smallest exponent */
    double q = ldexp(a, mant - E); /* exact: scaling by a power of two */
    double r = nearbyint(q);       /* default rounding mode: to nearest, ties to even */
    const double one = ldexp(1.0, mant);
    if (r >= 2.0 * one) { /* rounded up into the next binade */
        r *= 0.5;
        E += 1;
    }
    if (E > emax) return (uint16_t)(sign | exp_all);
    if (r < one) /* subnormal (only reachable with E == emin) */
        return (uint16_t)(sign | (uint16_t)r);
    uint16_t biased = (uint16_t)(E + bias);
    uint16_t frac = (uint16_t)(r - one);
    return (uint16_t)(sign | (uint16_t)(biased << mant) | frac);
}

uint16_t ref_double_to_f16_bits(double x) { return ref_encode_small_float(x, 10, 5); }
uint16_t ref_double_to_bf16_bits(double x) { return ref_encode_small_float(x, 7, 8); }

static int ref_elt_size(int dtype) {
    switch (dtype) {
        case REF_F32: return 4;
        case REF_F16: return 2;
        case REF_BF16: return 2;
        default: return 0;
    }
}

/* Element `idx` of a buffer stored in `dtype`, as a double. */
static double ref_load(const void* base, int64_t idx, int dtype) {
    if (dtype == REF_F32) {
        float f;
        memcpy(&f, (const char*)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + idx * 2, 2);
    return dtype == REF_F16 ? ref_f16_bits_to_double(h) : ref_bf16_bits_to_double(h);
}

/* Decode `n` stored elements of `dtype` to doubles. */
int ref_to_double(const void* in, int64_t n, int dtype, double* out) {
    if (ref_elt_size(dtype) == 0) return REF_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = ref_load(in, i, dtype);
    return REF_OK;
}

/* Round `n` doubles to `dtype` (round to nearest even) into `out`. */
int ref_cast(const double* in, int64_t n, int dtype, void* out) {
    if (ref_elt_size(dtype) == 0) return REF_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == REF_F32) {
            float f = (float)in[i]; /* C conversion rounds to nearest even */
            memcpy((char*)out + i * 4, &f, 4);
        } else {
            uint16_t h = dtype == REF_F16 ? ref_double_to_f16_bits(in[i])
                                          : ref_double_to_bf16_bits(in[i]);
            memcpy((char*)out + i * 2, &h, 2);
        }
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Address translation ("The one formula").                                  */
/* ------------------------------------------------------------------------ */

/* Physical token slot of logical position i, given one sequence's table. */
int64_t ref_physical_slot(const int32_t* table_row, int32_t block_size, int64_t i) {
    return (int64_t)table_row[i / block_size] * block_size + (i % block_size);
}

/* Offset (in elements) of row (slot, kv head g) in a [blocks][B][Hkv][D] cache. */
static int64_t ref_row_offset(int64_t slot, int32_t n_kv_heads, int32_t g, int32_t head_dim) {
    return (slot * n_kv_heads + g) * (int64_t)head_dim;
}

/* ------------------------------------------------------------------------ */
/* Append: each sequence's new token goes to the slot of its position.       */
/* ------------------------------------------------------------------------ */

/*
 * k_new, v_new: [num_seqs][n_kv_heads][head_dim] in `dtype`.
 * positions[s]: logical index of sequence s's new token.
 * The raw bits are copied; nothing else in the caches changes.
 */
int ref_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
               int32_t num_blocks, int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
               int dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* positions, int32_t num_seqs) {
    const int esz = ref_elt_size(dtype);
    if (esz == 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1) return REF_EINVAL;
    const int64_t row_bytes = (int64_t)n_kv_heads * head_dim * esz;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t p = positions[s];
        const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
        if (p < 0 || p / block_size >= max_blocks_per_seq) return REF_EINVAL;
        const int64_t slot = ref_physical_slot(row, block_size, p);
        if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return REF_EINVAL;
        memcpy((char*)k_cache + slot * row_bytes, (const char*)k_new + s * row_bytes, row_bytes);
        memcpy((char*)v_cache + slot * row_bytes, (const char*)v_new + s * row_bytes, row_bytes);
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Copy-on-write, the data half ("How a serving engine actually works",      */
/* section "Copy-on-write, because you have used fork()"): a sequence about  */
/* to write into a block that others also hold takes a private block first. */
/* The tokens the shared block already holds for it (its first n rows) must  */
/* then exist in the private block too; the pages' counter simulation skips  */
/* this copy.                                                                */
/* ------------------------------------------------------------------------ */

/*
 * For every i < n_copies: rows 0 .. n_rows[i]-1 of physical block src[i] are
 * copied bit for bit to the same rows of block dst[i], all heads, in both
 * caches.  Row r of block b is slot b * B + r.  Every argument is checked
 * before anything is written: a block outside the pool or a row count outside
 * [0, B] rejects the whole call.
 */
int ref_copy_blocks(void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size,
                    int32_t n_kv_heads, int32_t head_dim, int dtype, const int32_t* src,
                    const int32_t* dst, const int32_t* n_rows, int32_t n_copies) {
    const int esz = ref_elt_size(dtype);
    if (esz == 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || n_copies < 0) return REF_EINVAL;
    for (int32_t i = 0; i < n_copies; ++i)
        if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks || n_rows[i] < 0 ||
            n_rows[i] > block_size)
            return REF_EINVAL;
    const int64_t row_bytes = (int64_t)n_kv_heads * head_dim * esz;
    for (int32_t i = 0; i < n_copies; ++i)
        for (int32_t r = 0; r < n_rows[i]; ++r) {
            const int64_t from = (int64_t)src[i] * block_size + r;
            const int64_t to = (int64_t)dst[i] * block_size + r;
            memcpy((char*)k_cache + to * row_bytes, (const char*)k_cache + from * row_bytes, row_bytes);
            memcpy((char*)v_cache + to * row_bytes, (const char*)v_cache + from * row_bytes, row_bytes);
        }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Gather (snowch ch08, "The measurement"): one sequence's cache as a        */
/* contiguous [n_kv_heads][length][head_dim] array, here in double.          */
/* ------------------------------------------------------------------------ */

int ref_gather(const void* cache, int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
               int dtype, const int32_t* table_row, int32_t length, double* out) {
    if (ref_elt_size(dtype) == 0) return REF_EINVAL;
    for (int32_t g = 0; g < n_kv_heads; ++g)
        for (int32_t i = 0; i < length; ++i) {
            int64_t base = ref_row_offset(ref_physical_slot(table_row, block_size, i), n_kv_heads,
                                          g, head_dim);
            for (int32_t d = 0; d < head_dim; ++d)
                out[((int64_t)g * length + i) * head_dim + d] = ref_load(cache, base + d, dtype);
        }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode attention.                                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void* q; /* [S][Hq][D] */
    const void* k_cache;
    const void* v_cache;
    int32_t block_size, n_kv_heads, head_dim, dtype;
    const int32_t* block_tables; /* [S][max_blocks_per_seq] */
    int32_t max_blocks_per_seq;
    const int32_t* context_lens; /* [S] */
    int32_t n_q_heads;
    double scale;
} ref_problem;

/* scores z_i = scale * <q_h, K_i> for i < L, kv head g = h / (Hq / Hkv). */
static void ref_scores(const ref_problem* P, int32_t s, int32_t h, double* z) {
    const int32_t L = P->context_lens[s];
    const int32_t D = P->head_dim;
    const int32_t g = h / (P->n_q_heads / P->n_kv_heads);
    const int32_t* row = P->block_tables + (int64_t)s * P->max_blocks_per_seq;
    const int64_t qoff = ((int64_t)s * P->n_q_heads + h) * D;
    for (int32_t i = 0; i < L; ++i) {
        int64_t koff = ref_row_offset(ref_physical_slot(row, P->block_size, i), P->n_kv_heads, g, D);
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
            dot += ref_load(P->q, qoff + d, P->dtype) * ref_load(P->k_cache, koff + d, P->dtype);
        z[i] = P->scale * dot;
    }
}

/* out_row[d] = sum_{i in [lo,hi)} w_i * V_i[d]  with w_i = exp(z_i - m). */
static double ref_weighted_values(const ref_problem* P, int32_t s, int32_t h, const double* z,
                                  int32_t lo, int32_t hi, double m, double* out_row) {
    const int32_t D = P->head_dim;
    const int32_t g = h / (P->n_q_heads / P->n_kv_heads);
    const int32_t* row = P->block_tables + (int64_t)s * P->max_blocks_per_seq;
    double sum_w = 0.0;
    for (int32_t d = 0; d < D; ++d) out_row[d] = 0.0;
    for (int32_t i = lo; i < hi; ++i) {
        double w = exp(z[i] - m);
        sum_w += w;
        int64_t voff = ref_row_offset(ref_physical_slot(row, P->block_size, i), P->n_kv_heads, g, D);
        for (int32_t d = 0; d < D; ++d) out_row[d] += w * ref_load(P->v_cache, voff + d, P->dtype);
    }
    return sum_w;
}

/*
 * Plain softmax attention for one (sequence, query head): two passes, max
 * subtraction for range only (it does not change the exact value).  No causal
 * mask: the decode query attends to all L cached tokens, its own included.
 * L = 0 (the pages never produce it) gives an all-zero row.
 */
static void ref_decode_one(const ref_problem* P, int32_t s, int32_t h, double* z, double* out_row) {
    const int32_t L = P->context_lens[s];
    const int32_t D = P->head_dim;
    if (L <= 0) {
        for (int32_t d = 0; d < D; ++d) out_row[d] = 0.0;
        return;
    }
    ref_scores(P, s, h, z);
    double m = -INFINITY;
    for (int32_t i = 0; i < L; ++i) m = z[i] > m ? z[i] : m;
    double sum_w = ref_weighted_values(P, s, h, z, 0, L, m, out_row);
    for (int32_t d = 0; d < D; ++d) out_row[d] /= sum_w;
}

/*
 * Split-K form of the same quantity: the L tokens are cut into partitions
 * [jP, min((j+1)P, L)); each partition keeps (m_j, l_j, o_j) with
 * m_j = max z, l_j = sum exp(z - m_j), o_j = sum exp(z - m_j) V / l_j, and the
 * partitions are combined by the log-sum-exp rule
 *   M = max_j m_j,  out = sum_j l_j e^(m_j - M) o_j / sum_j l_j e^(m_j - M).
 * In exact arithmetic this equals ref_decode_one for every P.
 */
static void ref_decode_one_split(const ref_problem* P, int32_t s, int32_t h, int32_t part_tokens,
                                 double* z, double* o_part, double* out_row) {
    const int32_t L = P->context_lens[s];
    const int32_t D = P->head_dim;
    for (int32_t d = 0; d < D; ++d) out_row[d] = 0.0;
    if (L <= 0) return;
    ref_scores(P, s, h, z);
    const int32_t n_parts = (L + part_tokens - 1) / part_tokens;
    double* m = (double*)malloc(sizeof(double) * n_parts);
    double* l = (double*)malloc(sizeof(double) * n_parts);
    double* o = (double*)malloc(sizeof(double) * (size_t)n_parts * D);
    for (int32_t j = 0; j < n_parts; ++j) {
        int32_t lo = j * part_tokens;
        int32_t hi = lo + part_tokens < L ? lo + part_tokens : L;
        m[j] = -INFINITY;
        for (int32_t i = lo; i < hi; ++i) m[j] = z[i] > m[j] ? z[i] : m[j];
        l[j] = ref_weighted_values(P, s, h, z, lo, hi, m[j], o_part);
        for (int32_t d = 0; d < D; ++d) o[(int64_t)j * D + d] = o_part[d] / l[j];
    }
    double M = -INFINITY;
    for (int32_t j = 0; j < n_parts; ++j) M = m[j] > M ? m[j] : M;
    double den = 0.0;
    for (int32_t j = 0; j < n_parts; ++j) {
        double w = l[j] * exp(m[j] - M);
        den += w;
        for (int32_t d = 0; d < D; ++d) out_row[d] += w * o[(int64_t)j * D + d];
    }
    for (int32_t d = 0; d < D; ++d) out_row[d] /= den;
    free(m);
    free(l);
    free(o);
}

static int ref_check_problem(const ref_problem* P, int32_t num_seqs) {
    if (ref_elt_size(P->dtype) == 0 || P->block_size < 1 || P->n_kv_heads < 1 ||
        P->head_dim < 1 || P->n_q_heads < 1 || P->n_q_heads % P->n_kv_heads != 0)
        return REF_EINVAL;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t L = P->context_lens[s];
        if (L < 0 || (int64_t)L > (int64_t)P->max_blocks_per_seq * P->block_size) return REF_EINVAL;
    }
    return REF_OK;
}

/*
 * out: [num_seqs][n_q_heads][head_dim] doubles.  If seq_ids is non-NULL only
 * the n_ids listed sequences are computed (their rows of out are written, the
 * others left untouched); this lets the tests check sampled sequences of
 * workloads too large to compute whole on the CPU.  part_tokens > 0 selects
 * the split-K form with that partition length; 0 selects the plain form.
 */
int ref_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                         int32_t block_size, int32_t n_kv_heads, int32_t head_dim, int dtype,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                         double scale, const int32_t* seq_ids, int32_t n_ids, int32_t part_tokens,
                         double* out) {
    ref_problem P = {q, k_cache, v_cache, block_size, n_kv_heads, head_dim, dtype,
                     block_tables, max_blocks_per_seq, context_lens, n_q_heads, scale};
    if (ref_check_problem(&P, num_seqs) != REF_OK || part_tokens < 0) return REF_EINVAL;
    const int32_t n_sel = seq_ids ? n_ids : num_seqs;
    for (int32_t k = 0; k < n_sel; ++k)
        if (seq_ids && (seq_ids[k] < 0 || seq_ids[k] >= num_seqs)) return REF_EINVAL;
    int32_t max_len = 1;
    for (int32_t s = 0; s < num_seqs; ++s) max_len = context_lens[s] > max_len ? context_lens[s] : max_len;
    const int64_t n_work = (int64_t)n_sel * n_q_heads;

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * max_len);
        double* o_part = (double*)malloc(sizeof(double) * head_dim);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < n_work; ++w) {
            int32_t s = seq_ids ? seq_ids[w / n_q_heads] : (int32_t)(w / n_q_heads);
            int32_t h = (int32_t)(w % n_q_heads);
            double* out_row = out + ((int64_t)s * n_q_heads + h) * head_dim;
            if (part_tokens > 0)
                ref_decode_one_split(&P, s, h, part_tokens, z, o_part, out_row);
            else
                ref_decode_one(&P, s, h, z, out_row);
        }
        free(z);
        free(o_part);
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Swap ("How a serving engine actually works", section "When there are no   */
/* free blocks left"; "Paged Attention and the Block Manager", "Running out  */
/* of memory becomes a scheduling decision"): a preempted sequence's cache is */
/* copied to host memory, all of it, and later back into whatever blocks the */
/* allocator hands out then.  Slot i of the host buffer holds block blocks[i]. */
/* ------------------------------------------------------------------------ */

/*
 * Swap out: host_k[i] = k_cache[blocks[i]] (whole blocks: B rows of all heads),
 * and likewise for v; host buffers are [n][B][n_kv_heads][head_dim].  Swap in
 * (to_cache != 0): k_cache[blocks[i]] = host_k[i].  Bit copies; every block
 * index is checked before anything is written.
 */
int ref_swap(void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
             int32_t head_dim, int dtype, const int32_t* blocks, int32_t n, void* host_k, void* host_v,
             int to_cache) {
    const int esz = ref_elt_size(dtype);
    if (esz == 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || n < 0) return REF_EINVAL;
    for (int32_t i = 0; i < n; ++i)
        if (blocks[i] < 0 || blocks[i] >= num_blocks) return REF_EINVAL;
    const int64_t row_bytes = (int64_t)n_kv_heads * head_dim * esz;
    for (int32_t i = 0; i < n; ++i)
        for (int32_t r = 0; r < block_size; ++r) {
            const int64_t slot = (int64_t)blocks[i] * block_size + r; /* row r of the block */
            const int64_t h = (int64_t)i * block_size + r;            /* row r of host slot i */
            if (to_cache) {
                memcpy((char*)k_cache + slot * row_bytes, (const char*)host_k + h * row_bytes, row_bytes);
                memcpy((char*)v_cache + slot * row_bytes, (const char*)host_v + h * row_bytes, row_bytes);
            } else {
                memcpy((char*)host_k + h * row_bytes, (const char*)k_cache + slot * row_bytes, row_bytes);
                memcpy((char*)host_v + h * row_bytes, (const char*)v_cache + slot * row_bytes, row_bytes);
            }
        }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Chunked prefill ("How a serving engine actually works", section "Prefill  */
/* and decode are two different jobs": a long prompt is processed a slice at */
/* a time; "Paged Attention and the Block Manager", section "The build":     */
/* the table grows by as many blocks as n new tokens need).  A sequence whose */
/* cache holds L tokens after this step received its last n of them in the   */
/* step: they are written at positions L-n .. L-1, and the query of token j  */
/* of the chunk (position L-n+j) attends to positions 0 .. L-n+j -- the whole */
/* earlier context and the chunk up to itself.  n = 1 is a decode step.      */
/* ------------------------------------------------------------------------ */

/*
 * n-token append: rows cu_new[s] .. cu_new[s+1]-1 of k_new / v_new
 * ([total][n_kv_heads][head_dim]) go to the slots of positions start_pos[s],
 * start_pos[s] + 1, ... of sequence s.  Raw bits are copied; nothing else in
 * the caches changes.  Every position and block is checked before anything
 * is written.
 */
int ref_append_tokens(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      int32_t num_blocks, int32_t block_size, int32_t n_kv_heads, int32_t head_dim,
                      int dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* cu_new, const int32_t* start_pos, int32_t num_seqs) {
    const int esz = ref_elt_size(dtype);
    if (esz == 0 || block_size < 1 || n_kv_heads < 1 || head_dim < 1 || num_seqs < 0 || cu_new[0] != 0)
        return REF_EINVAL;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (cu_new[s + 1] < cu_new[s] || start_pos[s] < 0) return REF_EINVAL;
        const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int32_t j = cu_new[s]; j < cu_new[s + 1]; ++j) {
            const int64_t p = (int64_t)start_pos[s] + (j - cu_new[s]);
            if (p / block_size >= max_blocks_per_seq) return REF_EINVAL;
            const int64_t slot = ref_physical_slot(row, block_size, p);
            if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return REF_EINVAL;
        }
    }
    const int64_t row_bytes = (int64_t)n_kv_heads * head_dim * esz;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int32_t j = cu_new[s]; j < cu_new[s + 1]; ++j) {
            const int64_t slot = ref_physical_slot(row, block_size, (int64_t)start_pos[s] + (j - cu_new[s]));
            memcpy((char*)k_cache + slot * row_bytes, (const char*)k_new + j * row_bytes, row_bytes);
            memcpy((char*)v_cache + slot * row_bytes, (const char*)v_new + j * row_bytes, row_bytes);
        }
    }
    return REF_OK;
}

/*
 * One query row: q at element qoff ([D]), KV head g of sequence s, keys at
 * positions 0 .. n_keys-1; plain two-pass softmax in double.
 */
static void ref_prefill_one(const ref_problem* P, int32_t s, int64_t qoff, int32_t g, int32_t n_keys,
                            double* z, double* out_row) {
    const int32_t D = P->head_dim;
    const int32_t* row = P->block_tables + (int64_t)s * P->max_blocks_per_seq;
    double m = -INFINITY;
    for (int32_t i = 0; i < n_keys; ++i) {
        int64_t koff = ref_row_offset(ref_physical_slot(row, P->block_size, i), P->n_kv_heads, g, D);
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
            dot += ref_load(P->q, qoff + d, P->dtype) * ref_load(P->k_cache, koff + d, P->dtype);
        z[i] = P->scale * dot;
        m = z[i] > m ? z[i] : m;
    }
    double sum_w = 0.0;
    for (int32_t d = 0; d < D; ++d) out_row[d] = 0.0;
    for (int32_t i = 0; i < n_keys; ++i) {
        double w = exp(z[i] - m);
        sum_w += w;
        int64_t voff = ref_row_offset(ref_physical_slot(row, P->block_size, i), P->n_kv_heads, g, D);
        for (int32_t d = 0; d < D; ++d) out_row[d] += w * ref_load(P->v_cache, voff + d, P->dtype);
    }
    for (int32_t d = 0; d < D; ++d) out_row[d] /= sum_w;
}

/*
 * Prefill attention.  q, out: [total][n_q_heads][head_dim] (out in double),
 * total = cu_q[num_seqs]; sequence s owns query rows cu_q[s] .. cu_q[s+1]-1,
 * n_s of them, which are its last n_s tokens: row cu_q[s] + j sits at
 * position L_s - n_s + j and attends to positions 0 .. L_s - n_s + j.
 * Requires n_s <= L_s <= max_blocks_per_seq * block_size.  If row_ids is
 * non-NULL only those n_rows query rows are computed (the others are left
 * untouched), for sampled checks of large problems.
 */
int ref_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                          int32_t block_size, int32_t n_kv_heads, int32_t head_dim, int dtype,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q,
                          const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                          double scale, const int32_t* row_ids, int32_t n_rows, double* out) {
    ref_problem P = {q, k_cache, v_cache, block_size, n_kv_heads, head_dim, dtype,
                     block_tables, max_blocks_per_seq, context_lens, n_q_heads, scale};
    if (ref_check_problem(&P, num_seqs) != REF_OK || num_seqs < 0 || cu_q[0] != 0) return REF_EINVAL;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (cu_q[s + 1] < cu_q[s] || cu_q[s + 1] - cu_q[s] > context_lens[s]) return REF_EINVAL;
    const int64_t total = cu_q[num_seqs];
    const int64_t n_sel = row_ids ? n_rows : total;
    for (int64_t k = 0; k < n_sel; ++k)
        if (row_ids && (row_ids[k] < 0 || row_ids[k] >= total)) return REF_EINVAL;
    int32_t max_len = 1;
    for (int32_t s = 0; s < num_seqs; ++s) max_len = context_lens[s] > max_len ? context_lens[s] : max_len;
    const int32_t group = n_q_heads / n_kv_heads;

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * max_len);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < n_sel * n_q_heads; ++w) {
            const int64_t t = row_ids ? row_ids[w / n_q_heads] : w / n_q_heads;
            const int32_t h = (int32_t)(w % n_q_heads);
            int32_t s = 0;
            while (cu_q[s + 1] <= t) ++s; /* the sequence owning query row t */
            const int32_t n = cu_q[s + 1] - cu_q[s];
            const int32_t pos = context_lens[s] - n + (int32_t)(t - cu_q[s]);
            ref_prefill_one(&P, s, (t * n_q_heads + h) * head_dim, h / group, pos + 1, z,
                            out + (t * n_q_heads + h) * head_dim);
        }
        free(z);
    }
    return REF_OK;
}

/* Number of OpenMP threads the oracle runs with (for reporting). */
int ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
