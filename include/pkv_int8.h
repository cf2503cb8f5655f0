/*
 * pkv_int8.h - INT8 KV cache for libpkv: a quantising kv_append, decode
 * over the INT8 cache, and the two in one launch.
 *
 * "从零搭建AI工程能力：手写KV Cache与动态批处理实战" section 3.2 keeps the KV
 * cache as 8-bit integers instead of 16-bit floats: half the memory, and half
 * the bytes a decode step streams from HBM, at the cost of a quantisation
 * error that every later step reads again.  The page names no scheme; this
 * library uses symmetric absmax quantisation with one fp32 scale per
 * (token, KV head) row, which suits rows that arrive one at a time (a block's
 * earlier rows never need requantising):
 *
 *   scale   = max_d |x_d| / 127                     (fp32, IEEE division)
 *   code_d  = round_to_nearest_even(x_d / scale)    (fp32 quotient; in [-127, 127])
 *   x_d    ~= code_d * scale                        (an all-zero row: scale 0, codes 0)
 *
 * Layout, next to the bf16 pools of pkv.h:
 *   k_codes, v_codes    [num_blocks][num_kv_heads][block_size][head_dim] int8
 *   k_scales, v_scales  [num_blocks][num_kv_heads][block_size] fp32 (one per slot)
 * so the codes of a tile of keys are contiguous and its scales are one
 * contiguous row.  Conventions (device pointers owned by the caller, streams,
 * status codes, block tables, supported head sizes and GQA groups) are those
 * of pkv.h, except that block_size is a power of two in [32, 256].  Inputs
 * must be finite.
 */
#ifndef PKV_INT8_H
#define PKV_INT8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * kv_append_int8: quantise new K/V rows and write codes and scales into the
 * INT8 cache at the positions pkv_kv_append would use (section 4.3.1 of
 * "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎").  Arguments as for pkv_kv_append,
 * with the two code pools and the two scale arrays in place of the bf16
 * pools; the same preconditions, and rows breaking them are skipped.
 */
int32_t pkv_kv_append_int8(int8_t* k_codes, int8_t* v_codes, float* k_scales, float* v_scales,
                           const uint16_t* k_new, const uint16_t* v_new,
                           const int32_t* cu_new_lens, const int32_t* ctx_lens,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t num_seqs, int32_t total_new_tokens, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           void* stream);

/*
 * Bytes of device workspace pkv_paged_gqa_decode_int8 needs (its split plan
 * differs from the bf16 decode's).  Returns 0 for unsupported shapes.  As for
 * the bf16 decode, the workspace is zero-filled before its first use, and one
 * workspace may serve both formats.
 */
size_t pkv_decode_int8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_seq_len, int64_t total_kv_tokens);

/*
 * paged_gqa_decode_int8: pkv_paged_gqa_decode over the INT8 cache, every key
 * and value row read as code * scale (q and out stay bf16).  Arguments as for
 * pkv_paged_gqa_decode with the codes and scales in place of the bf16 pools
 * and a workspace of pkv_decode_int8_workspace_bytes(...).  Rows past a
 * sequence's length may hold anything (NaN scales included).
 */
int32_t pkv_paged_gqa_decode_int8(uint16_t* out, const uint16_t* q,
                                  const int8_t* k_codes, const int8_t* v_codes,
                                  const float* k_scales, const float* v_scales,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  float scale, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * paged_gqa_decode_append_int8: one decode step over the INT8 cache in one
 * launch -- pkv_kv_append_int8 of one new row per sequence followed by
 * pkv_paged_gqa_decode_int8, as pkv_paged_gqa_decode_append does for bf16.
 *
 *   k_new, v_new     [num_seqs][num_kv_heads][head_dim] bf16: the row of
 *                    position seq_lens[s] - 1 of each sequence (a sequence
 *                    with seq_lens[s] == 0 appends nothing and yields zeros)
 *   k_codes ... v_scales  written at that position (codes and scales equal
 *                    to pkv_kv_append_int8's)
 *   other arguments  as for pkv_paged_gqa_decode_int8 (same workspace size)
 *
 * The outputs equal pkv_kv_append_int8 followed by pkv_paged_gqa_decode_int8
 * up to summation order.  Preconditions as for both: the new rows' slots
 * belong to their sequence alone.
 */
int32_t pkv_paged_gqa_decode_append_int8(uint16_t* out, const uint16_t* q,
                                         const uint16_t* k_new, const uint16_t* v_new,
                                         int8_t* k_codes, int8_t* v_codes, float* k_scales, float* v_scales,
                                         const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, void* workspace, size_t workspace_bytes,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_INT8_H */
