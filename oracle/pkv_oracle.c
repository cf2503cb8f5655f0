/*
 * CPU oracle for paged-KV causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file, and everything under oracle/, is
 * called only by the tests, by the smoke check and by the CPU-baseline leg of
 * the benchmark.  The product path (the HIP library) never links, loads or
 * calls it, and it shares no code, header or table with that library.
 *
 * It is deliberately plain and slow: fp64 arithmetic, one query row at a time,
 * keys gathered one by one through the block table in logical order.
 *
 * What it computes, and where the pages define it:
 *
 *  - oracle_kv_append: the paged write of new K/V rows.  "扔掉 vLLM！从零构建
 *    Qwen3-8B 推理引擎" section 4.3.1 keeps the KV cache as fixed-size blocks
 *    (256 tokens) taken from a pool, each with separate K and V and a fill
 *    count, and appends a sequence's new rows into its last block, opening a
 *    new block when that one is full.  So logical position pos of a sequence
 *    lives in the sequence's block pos / B at slot pos % B.  "从零搭建AI工程能力：
 *    手写KV Cache与动态批处理实战" (the SimpleKVCache listing in section 4) writes
 *    the new rows at the current length and keeps a [heads][seq][dim] order
 *    inside the buffer, which is the per-block order used here:
 *    pool[block][kv_head][slot][dim].
 *
 *  - oracle_attention / oracle_attention_rows: softmax(Q K^T * scale) V with a
 *    causal mask, as "从零手搓AI推理引擎：避开调包陷阱的工程实践指南" section 2.2
 *    defines it: each position sees itself and the positions before it
 *    (inclusive diagonal), and the softmax subtracts the row maximum before
 *    exponentiating.  The scale is an argument (the pages use 1/sqrt(head_dim)).
 *    Query heads are grouped as in page 1 section 4.4.2: query head h reads KV
 *    head h / (Hq / Hkv), i.e. consecutive query heads share one KV head.
 *    A query row r of a chunk of n rows appended to a sequence of final length
 *    L sits at absolute position L - n + r (chunked prefill, page 3 section 3.3;
 *    decode is the case n = 1).  Masked keys are left out of the softmax; the
 *    pages' additive -1e9 mask gives exactly the same result in fp64 because at
 *    least one key (the diagonal) is never masked.  The pages never meet a row
 *    with no key at all (a decode row of an empty sequence, L = 0); such a row
 *    is defined here as all zeros.
 *
 *  - oracle_quantize_int8 / oracle_kv_append_int8 / oracle_attention_rows_int8:
 *    the INT8 KV cache of "从零搭建AI工程能力：手写KV Cache与动态批处理实战"
 *    section 3.2 (the cache kept as 8-bit integers instead of 16-bit floats,
 *    half the memory, with a quantisation error that every later step reads
 *    again).  The page names no scheme; the reading taken here is the plainest
 *    one that suits rows arriving one at a time: symmetric absmax quantisation
 *    with one fp32 scale per (token, KV head) row, scale = max|x| / 127 and
 *    code = x / scale rounded to the nearest integer (ties to even), so that
 *    x is approximated by code * scale.  An all-zero row has scale 0 and
 *    codes 0.  The quantiser runs in fp32 (IEEE division and rounding), the
 *    precision in which both this oracle and the HIP path take the integer
 *    decision; attention then reads the dequantised values code * scale,
 *    which are exact in fp64.
 *
 *  - oracle_qkv_project_append: the fused QKV projection of "扔掉 vLLM！从零构建
 *    Qwen3-8B 推理引擎" section 4.4.3 (the q, k and v linear projections as one
 *    matmul against the merged weight, whose output is cut into q, k and v),
 *    with the k and v parts placed in the paged cache as oracle_kv_append
 *    places new rows.  The page stops at the three slices; storing k and v in
 *    the cache straight from the projection is this repository's reading of
 *    the fused step (the slices would be appended next anyway).  No bias and
 *    no position encoding: the page's projection has neither.  Each output is
 *    the dot product of a new row with a row of the merged weight, summed in
 *    fp64 (bf16 products are exact in fp64) and rounded once to bf16, to
 *    nearest with ties to even.
 *
 * bf16 inputs are widened exactly: the 16 bits become the top half of an IEEE
 * binary32 word, which is then converted to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS (-1)
#define ORACLE_ERR_BLOCK (-2)     /* a block id outside [0, num_blocks) or a position past the table */
#define ORACLE_ERR_DUP_SLOT (-3)  /* two new rows target the same slot */
#define ORACLE_ERR_OOM (-4)

static float bf16_to_float(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static double bf16_to_double(uint16_t h) { return (double)bf16_to_float(h); }

/* Sequence that owns packed row t, given cu[0..S] with cu[0] = 0. */
static int owner_of_row(const int32_t* cu, int num_seqs, int t) {
    int s = 0;
    while (s + 1 < num_seqs && cu[s + 1] <= t) ++s;
    return s;
}

/*
 * Where packed new row t goes: position ctx_lens[s] + (t - cu_new_lens[s]) of
 * its sequence s, i.e. block block_table[s][pos / B], slot pos % B.
 */
static int target_slot(const int32_t* cu_new_lens, const int32_t* ctx_lens, const int32_t* block_table,
                       int max_blocks_per_seq, int num_seqs, int block_size, int num_blocks, int t,
                       int* blk_out, long* slot_out) {
    int s = owner_of_row(cu_new_lens, num_seqs, t);
    long pos = (long)ctx_lens[s] + (t - cu_new_lens[s]);
    long lblock = pos / block_size;
    long slot = pos % block_size;
    if (pos < 0 || lblock >= max_blocks_per_seq) return ORACLE_ERR_BLOCK;
    int blk = block_table[(size_t)s * max_blocks_per_seq + lblock];
    if (blk < 0 || blk >= num_blocks) return ORACLE_ERR_BLOCK;
    *blk_out = blk;
    *slot_out = slot;
    return ORACLE_OK;
}

int oracle_kv_append(uint16_t* k_pool, uint16_t* v_pool,
                     const uint16_t* k_new, const uint16_t* v_new,
                     const int32_t* cu_new_lens, const int32_t* ctx_lens,
                     const int32_t* block_table, int max_blocks_per_seq,
                     int num_seqs, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return ORACLE_ERR_ARGS;
    const int total = num_seqs > 0 ? cu_new_lens[num_seqs] : 0;
    /* one flag per physical slot, to catch two rows aimed at the same slot */
    size_t nslots = (size_t)num_blocks * (size_t)block_size;
    unsigned char* written = (unsigned char*)calloc(nslots ? nslots : 1, 1);
    if (!written) return ORACLE_ERR_OOM;
    int rc = ORACLE_OK;
    for (int t = 0; t < total && rc == ORACLE_OK; ++t) {
        int blk;
        long slot;
        rc = target_slot(cu_new_lens, ctx_lens, block_table, max_blocks_per_seq, num_seqs, block_size,
                         num_blocks, t, &blk, &slot);
        if (rc != ORACLE_OK) break;
        size_t flag = (size_t)blk * block_size + slot;
        if (written[flag]) { rc = ORACLE_ERR_DUP_SLOT; break; }
        written[flag] = 1;
        for (int g = 0; g < num_kv_heads; ++g) {
            size_t dst = (((size_t)blk * num_kv_heads + g) * block_size + slot) * head_dim;
            size_t src = ((size_t)t * num_kv_heads + g) * head_dim;
            memcpy(k_pool + dst, k_new + src, (size_t)head_dim * sizeof(uint16_t));
            memcpy(v_pool + dst, v_new + src, (size_t)head_dim * sizeof(uint16_t));
        }
    }
    free(written);
    return rc;
}

/*
 * Symmetric absmax quantisation of one row of head_dim bf16 values to INT8
 * ("从零搭建AI工程能力：手写KV Cache与动态批处理实战" section 3.2, with the
 * reading stated at the top of this file), in fp32.
 */
void oracle_quantize_int8(int8_t* codes, float* scale_out, const uint16_t* row, int head_dim) {
    float amax = 0.0f;
    for (int d = 0; d < head_dim; ++d) {
        float a = fabsf(bf16_to_float(row[d]));
        if (a > amax) amax = a;
    }
    float scale = amax / 127.0f;
    for (int d = 0; d < head_dim; ++d) {
        float c = scale > 0.0f ? rintf(bf16_to_float(row[d]) / scale) : 0.0f;
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        codes[d] = (int8_t)c;
    }
    *scale_out = scale;
}

/*
 * kv_append into an INT8 cache: the same placement as oracle_kv_append, each
 * new (token, KV head) row quantised on the way in.  Pools are
 * [num_blocks][num_kv_heads][block_size][head_dim] int8 codes and
 * [num_blocks][num_kv_heads][block_size] fp32 scales.
 */
int oracle_kv_append_int8(int8_t* k_codes, int8_t* v_codes, float* k_scales, float* v_scales,
                          const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* cu_new_lens, const int32_t* ctx_lens,
                          const int32_t* block_table, int max_blocks_per_seq,
                          int num_seqs, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return ORACLE_ERR_ARGS;
    const int total = num_seqs > 0 ? cu_new_lens[num_seqs] : 0;
    size_t nslots = (size_t)num_blocks * (size_t)block_size;
    unsigned char* written = (unsigned char*)calloc(nslots ? nslots : 1, 1);
    if (!written) return ORACLE_ERR_OOM;
    int rc = ORACLE_OK;
    for (int t = 0; t < total && rc == ORACLE_OK; ++t) {
        int blk;
        long slot;
        rc = target_slot(cu_new_lens, ctx_lens, block_table, max_blocks_per_seq, num_seqs, block_size,
                         num_blocks, t, &blk, &slot);
        if (rc != ORACLE_OK) break;
        if (written[(size_t)blk * block_size + slot]) { rc = ORACLE_ERR_DUP_SLOT; break; }
        written[(size_t)blk * block_size + slot] = 1;
        for (int g = 0; g < num_kv_heads; ++g) {
            size_t row = ((size_t)blk * num_kv_heads + g) * block_size + slot;
            size_t src = ((size_t)t * num_kv_heads + g) * head_dim;
            oracle_quantize_int8(k_codes + row * head_dim, k_scales + row, k_new + src, head_dim);
            oracle_quantize_int8(v_codes + row * head_dim, v_scales + row, v_new + src, head_dim);
        }
    }
    free(written);
    return rc;
}

/*
 * A double rounded once to bf16, to nearest with ties to even (bf16 keeps 8
 * significant bits; below 2^-126 its spacing stays 2^-133; past the largest
 * finite value it is infinite).
 */
static uint16_t double_to_bf16(double v) {
    if (v != v) return 0x7FC0;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m 2^e, m in [0.5, 1): spacing 2^(e - 8) */
    int q = e - 8;
    if (q < -133) q = -133;
    const double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r >= 0x1p128) return sign | 0x7F80;
    const float f = (float)r;           /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return sign | (uint16_t)(bits >> 16);
}

int oracle_qkv_project_append(uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool,
                              const uint16_t* x, const uint16_t* w,
                              const int32_t* cu_new_lens, const int32_t* ctx_lens,
                              const int32_t* block_table, int max_blocks_per_seq,
                              int num_seqs, int d_model, int num_q_heads, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks) {
    if (num_seqs < 0 || d_model <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks < 0)
        return ORACLE_ERR_ARGS;
    const int total = num_seqs > 0 ? cu_new_lens[num_seqs] : 0;
    const int nq = num_q_heads * head_dim, nkv = num_kv_heads * head_dim;
    const int n_out = nq + 2 * nkv;    /* rows of the merged weight: q, then k, then v features */
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n_out ? n_out : 1));
    size_t nslots = (size_t)num_blocks * (size_t)block_size;
    unsigned char* written = (unsigned char*)calloc(nslots ? nslots : 1, 1);
    if (!y || !written) {
        free(y);
        free(written);
        return ORACLE_ERR_OOM;
    }
    int rc = ORACLE_OK;
    for (int t = 0; t < total && rc == ORACLE_OK; ++t) {
        const uint16_t* xt = x + (size_t)t * d_model;
        for (int n = 0; n < n_out; ++n) {
            const uint16_t* wn = w + (size_t)n * d_model;
            double acc = 0.0;
            for (int k = 0; k < d_model; ++k) acc += bf16_to_double(xt[k]) * bf16_to_double(wn[k]);
            y[n] = double_to_bf16(acc);
        }
        memcpy(q_out + (size_t)t * nq, y, sizeof(uint16_t) * (size_t)nq);
        int blk;
        long slot;
        rc = target_slot(cu_new_lens, ctx_lens, block_table, max_blocks_per_seq, num_seqs, block_size,
                         num_blocks, t, &blk, &slot);
        if (rc != ORACLE_OK) break;
        if (written[(size_t)blk * block_size + slot]) { rc = ORACLE_ERR_DUP_SLOT; break; }
        written[(size_t)blk * block_size + slot] = 1;
        for (int g = 0; g < num_kv_heads; ++g) {
            size_t dst = (((size_t)blk * num_kv_heads + g) * block_size + slot) * head_dim;
            memcpy(k_pool + dst, y + nq + (size_t)g * head_dim, sizeof(uint16_t) * (size_t)head_dim);
            memcpy(v_pool + dst, y + nq + nkv + (size_t)g * head_dim, sizeof(uint16_t) * (size_t)head_dim);
        }
    }
    free(y);
    free(written);
    return rc;
}

/*
 * A KV pool as attention reads it: bf16 rows, or INT8 codes with one fp32
 * scale per row.  Row index = (block * num_kv_heads + kv_head) * block_size + slot.
 */
typedef struct {
    const uint16_t* bf16;  /* [rows][head_dim], or NULL for an INT8 pool */
    const int8_t* codes;   /* [rows][head_dim] */
    const float* scales;   /* [rows] */
} kv_pool;

/* Element d of a pool row, as a double (an INT8 one dequantised: code * scale). */
static double kv_elem(const kv_pool* pool, size_t row, int head_dim, int d) {
    if (pool->bf16) return bf16_to_double(pool->bf16[row * head_dim + d]);
    return (double)pool->codes[row * head_dim + d] * (double)pool->scales[row];
}

/*
 * One output row: query head h of sequence s at absolute position p attends to
 * keys 0..p of that sequence.  out_row receives head_dim doubles.
 * Returns ORACLE_ERR_BLOCK if a needed block id is invalid.
 */
static int attend_one(double* out_row, const uint16_t* q_row,
                      const kv_pool* k_pool, const kv_pool* v_pool,
                      const int32_t* table_row, int max_blocks_per_seq,
                      int p, int kv_head, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, double scale,
                      double* z /* scratch, p+1 doubles */) {
    const int nkeys = p + 1;
    if (nkeys <= 0) { /* no key at or before this position: the row is zero */
        for (int d = 0; d < head_dim; ++d) out_row[d] = 0.0;
        return ORACLE_OK;
    }
    if ((nkeys - 1) / block_size >= max_blocks_per_seq) return ORACLE_ERR_BLOCK;
    /* scores z_j = scale * <q, k_j>, keys gathered through the block table */
    double zmax = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        int blk = table_row[j / block_size];
        if (blk < 0 || blk >= num_blocks) return ORACLE_ERR_BLOCK;
        size_t krow = ((size_t)blk * num_kv_heads + kv_head) * block_size + j % block_size;
        double dot = 0.0;
        for (int d = 0; d < head_dim; ++d) dot += bf16_to_double(q_row[d]) * kv_elem(k_pool, krow, head_dim, d);
        z[j] = scale * dot;
        if (z[j] > zmax) zmax = z[j];
    }
    /* stable softmax: subtract the maximum, exponentiate, normalise */
    double denom = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        z[j] = exp(z[j] - zmax);
        denom += z[j];
    }
    for (int d = 0; d < head_dim; ++d) out_row[d] = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        int blk = table_row[j / block_size];
        size_t vrow = ((size_t)blk * num_kv_heads + kv_head) * block_size + j % block_size;
        for (int d = 0; d < head_dim; ++d) out_row[d] += z[j] * kv_elem(v_pool, vrow, head_dim, d);
    }
    for (int d = 0; d < head_dim; ++d) out_row[d] /= denom;
    return ORACLE_OK;
}

static int check_heads(int hq, int hkv, int d, int bs) {
    return hq > 0 && hkv > 0 && hq % hkv == 0 && d > 0 && bs > 0;
}

/*
 * Selected output rows.  Item i is (sequence item_seq[i], query row item_row[i]
 * of that sequence's q_len_s = cu_q_lens[s+1]-cu_q_lens[s] rows, query head
 * item_head[i]); its result goes to out[i][0..head_dim).
 * q is packed [cu_q_lens[S]][Hq][D].  num_threads <= 0 uses the OpenMP default.
 */
static int attention_rows(double* out, int n_items,
                          const int32_t* item_seq, const int32_t* item_row, const int32_t* item_head,
                          const uint16_t* q, const int32_t* cu_q_lens,
                          const kv_pool* k_pool, const kv_pool* v_pool,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, int num_threads) {
    if (!check_heads(num_q_heads, num_kv_heads, head_dim, block_size) || n_items < 0) return ORACLE_ERR_ARGS;
    const int group = num_q_heads / num_kv_heads;
    int max_len = 1;
    for (int s = 0; s < num_seqs; ++s) if (seq_lens[s] > max_len) max_len = seq_lens[s];
    int rc = ORACLE_OK;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)max_len);
        if (!z) {
#pragma omp atomic write
            rc = ORACLE_ERR_OOM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n_items; ++i) {
            if (!z) continue;
            int s = item_seq[i], r = item_row[i], h = item_head[i];
            int n = cu_q_lens[s + 1] - cu_q_lens[s];
            if (s < 0 || s >= num_seqs || r < 0 || r >= n || h < 0 || h >= num_q_heads) {
#pragma omp atomic write
                rc = ORACLE_ERR_ARGS;
                continue;
            }
            int p = seq_lens[s] - n + r; /* absolute position of this query row; < 0 only if seq_len < n */
            const uint16_t* q_row = q + ((size_t)(cu_q_lens[s] + r) * num_q_heads + h) * head_dim;
            int e = attend_one(out + (size_t)i * head_dim, q_row, k_pool, v_pool,
                               block_table + (size_t)s * max_blocks_per_seq, max_blocks_per_seq,
                               p, h / group, num_kv_heads, head_dim, block_size, num_blocks,
                               (double)scale, z);
            if (e != ORACLE_OK) {
#pragma omp atomic write
                rc = e;
            }
        }
        free(z);
    }
    return rc;
}

int oracle_attention_rows(double* out, int n_items,
                          const int32_t* item_seq, const int32_t* item_row, const int32_t* item_head,
                          const uint16_t* q, const int32_t* cu_q_lens,
                          const uint16_t* k_pool, const uint16_t* v_pool,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, int num_threads) {
    kv_pool k = {k_pool, NULL, NULL}, v = {v_pool, NULL, NULL};
    return attention_rows(out, n_items, item_seq, item_row, item_head, q, cu_q_lens, &k, &v, block_table,
                          max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, scale, num_threads);
}

/*
 * The same rows over an INT8 cache (codes and per-row scales as written by
 * oracle_kv_append_int8), every key and value read as code * scale.
 */
int oracle_attention_rows_int8(double* out, int n_items,
                               const int32_t* item_seq, const int32_t* item_row, const int32_t* item_head,
                               const uint16_t* q, const int32_t* cu_q_lens,
                               const int8_t* k_codes, const int8_t* v_codes,
                               const float* k_scales, const float* v_scales,
                               const int32_t* block_table, int max_blocks_per_seq,
                               const int32_t* seq_lens, int num_seqs,
                               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, float scale, int num_threads) {
    kv_pool k = {NULL, k_codes, k_scales}, v = {NULL, v_codes, v_scales};
    return attention_rows(out, n_items, item_seq, item_row, item_head, q, cu_q_lens, &k, &v, block_table,
                          max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, scale, num_threads);
}

/*
 * Every output row: out is [cu_q_lens[S]][Hq][D] doubles, laid out like q.
 */
int oracle_attention(double* out, const uint16_t* q, const int32_t* cu_q_lens,
                     const uint16_t* k_pool, const uint16_t* v_pool,
                     const int32_t* block_table, int max_blocks_per_seq,
                     const int32_t* seq_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks, float scale, int num_threads) {
    if (!check_heads(num_q_heads, num_kv_heads, head_dim, block_size) || num_seqs < 0) return ORACLE_ERR_ARGS;
    const int total = num_seqs > 0 ? cu_q_lens[num_seqs] : 0;
    const size_t n_items = (size_t)total * num_q_heads;
    int32_t* it = (int32_t*)malloc(sizeof(int32_t) * 3 * (n_items ? n_items : 1));
    if (!it) return ORACLE_ERR_OOM;
    size_t i = 0;
    for (int s = 0; s < num_seqs; ++s)
        for (int r = 0; r < cu_q_lens[s + 1] - cu_q_lens[s]; ++r)
            for (int h = 0; h < num_q_heads; ++h, ++i) {
                it[i] = s;
                it[n_items + i] = r;
                it[2 * n_items + i] = h;
            }
    /* items are enumerated in the same order as the packed output rows */
    int rc = oracle_attention_rows(out, (int)n_items, it, it + n_items, it + 2 * n_items, q, cu_q_lens,
                                   k_pool, v_pool, block_table, max_blocks_per_seq, seq_lens, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                                   num_threads);
    free(it);
    return rc;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
