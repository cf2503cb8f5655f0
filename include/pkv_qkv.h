/*
 * pkv_qkv.h - the fused QKV projection of libpkv, whose epilogue writes the
 * k and v rows straight into the paged KV cache.
 *
 * "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.3 replaces the three
 * linear projections q = W_q x, k = W_k x, v = W_v x by one matmul against
 * the merged weight W = [W_q; W_k; W_v] and cuts its output into q, k and v;
 * the k and v rows are what kv_append then writes into the cache (section
 * 4.3.1).  pkv_qkv_project_append does both in one launch, so the k / v rows
 * are stored once, in their cache slots.  There is no bias and no position
 * encoding (the page's projection has neither).
 *
 * Conventions (device pointers owned by the caller, streams, status codes,
 * the pool layout and block tables, supported head sizes and GQA groups) are
 * those of pkv.h.
 */
#ifndef PKV_QKV_H
#define PKV_QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 *   q_out            [total_new_tokens][num_q_heads][head_dim] bf16, written
 *   k_pool, v_pool   [num_blocks][num_kv_heads][block_size][head_dim] bf16,
 *                    written at each token's slot
 *   x                [total_new_tokens][d_model] bf16: the new tokens' inputs,
 *                    packed in sequence order (d_model a multiple of 64)
 *   w_qkv            [(num_q_heads + 2 num_kv_heads) head_dim][d_model] bf16,
 *                    row-major: the q rows, then the k rows, then the v rows
 *                    (output feature h * head_dim + d of each part is head h,
 *                    dim d)
 *   cu_new_lens, ctx_lens, block_table, max_blocks_per_seq
 *                    as for pkv_kv_append: token t of sequence s goes to
 *                    position ctx_lens[s] + t
 *
 * Each output is the dot product of a token's x row with a row of w_qkv,
 * accumulated in fp32 and rounded to bf16 (nearest, ties to even).
 * Preconditions and the handling of tokens breaking them as for
 * pkv_kv_append (their k / v rows are not written; q is).  Sizes must keep
 * total_new_tokens * d_model and the rows of w_qkv times d_model below 2^30.
 */
int32_t pkv_qkv_project_append(uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool,
                               const uint16_t* x, const uint16_t* w_qkv,
                               const int32_t* cu_new_lens, const int32_t* ctx_lens,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               int32_t num_seqs, int32_t total_new_tokens, int32_t d_model,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_QKV_H */
