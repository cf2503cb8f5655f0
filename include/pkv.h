/*
 * pkv.h - paged-KV causal grouped-query attention for AMD MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Three operations, as the Qwen3-8B engine on the page
 * "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" uses them:
 *
 *   pkv_kv_append        scatter new K/V rows into fixed-size cache blocks
 *                        (section 4.3.1, the paged KV block manager);
 *   pkv_paged_gqa_decode one query row per sequence, several query heads
 *                        sharing one KV head (section 4.4.2);
 *   pkv_paged_gqa_prefill causal attention of a chunk of query rows over the
 *                        cached keys plus the chunk itself (section 4.4.1, and
 *                        chunked prefill on "从零搭建AI工程能力：手写KV Cache与
 *                        动态批处理实战" section 3.3).
 *
 * plus pkv_paged_gqa_decode_append, a decode step's append and decode in one
 * launch.
 *
 * Attention is softmax(Q K^T * scale) V with an inclusive causal mask, as
 * "从零手搓AI推理引擎：避开调包陷阱的工程实践指南" section 2.2 defines it.
 *
 * Common conventions
 * ------------------
 *  - bf16 tensors are passed as uint16_t bit patterns; int32 for indices.
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates nothing, frees nothing, keeps no pointer after a call returns
 *    and has no mutable global state (one exception:
 *    pkv_paged_gqa_decode_append_static's per-GPU static scratch); calls on
 *    different streams may run concurrently.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls validate their
 *    scalar arguments on the host, enqueue kernels on `stream` and return
 *    without synchronising; nothing is read back from the device.
 *  - KV pools: K and V are separate arrays of shape
 *      [num_blocks][num_kv_heads][block_size][head_dim]   (bf16)
 *    so one (block, kv head) tile is contiguous.
 *  - block_table: [num_seqs][max_blocks_per_seq] int32; logical position pos
 *    of sequence s lives in physical block block_table[s][pos / block_size]
 *    at slot pos % block_size.  Entries past a sequence's last block are never
 *    read.  Different sequences may map logical blocks to the same physical
 *    block (a shared prefix) for reading.
 *  - Query head h uses KV head h / (num_q_heads / num_kv_heads).
 *  - Supported: head_dim 64 or 128; block_size a power of two in [16, 256];
 *    num_q_heads / num_kv_heads in {1, 2, 4, 8}; pointers 16-byte aligned.
 *
 * Errors: a non-zero return means the arguments were rejected on the host and
 * nothing was launched or written (PKV_ERR_HIP: a launch failed; earlier
 * kernels of the same call may have run).  Device-array contents (block ids,
 * lengths) are preconditions: kernels never read or write outside the
 * arrays whose sizes the arguments give, but results for invalid contents
 * are unspecified.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

enum {
    PKV_OK = 0,
    PKV_ERR_NULL_POINTER = 1, /* a required pointer is NULL                       */
    PKV_ERR_BAD_SHAPE = 2,    /* sizes negative, inconsistent or unsupported      */
    PKV_ERR_MISALIGNED = 3,   /* a tensor pointer is not 16-byte aligned          */
    PKV_ERR_WORKSPACE = 4,    /* decode workspace missing or too small            */
    PKV_ERR_HIP = 5,          /* a kernel launch failed                           */
    PKV_ERR_SCRATCH_LIMIT = 8 /* the call needs more than the static decode scratch */
};

/* Returns PKV_ABI_VERSION. */
int32_t pkv_abi_version(void);

/* Static text for a status code (never NULL). */
const char* pkv_status_string(int32_t status);

/*
 * kv_append: write new K/V rows into the paged pools ("扔掉 vLLM！从零构建
 * Qwen3-8B 推理引擎" section 4.3.1: rows go into the sequence's current block,
 * a new block once it is full; page "从零搭建AI工程能力" section 4: writes start
 * at the current length).
 *
 *   k_pool, v_pool   [num_blocks][num_kv_heads][block_size][head_dim], written in place
 *   k_new, v_new     [total_new_tokens][num_kv_heads][head_dim], rows of all
 *                    sequences packed in sequence order
 *   cu_new_lens      [num_seqs + 1], cu_new_lens[0] = 0, cu_new_lens[num_seqs] = total_new_tokens;
 *                    rows cu_new_lens[s] .. cu_new_lens[s+1]-1 belong to sequence s
 *   ctx_lens         [num_seqs] tokens already cached: row t of sequence s goes
 *                    to position ctx_lens[s] + t
 *   block_table      [num_seqs][max_blocks_per_seq]
 *
 * A pure bit copy: each new row is copied unchanged.  Preconditions: every
 * target position is below max_blocks_per_seq * block_size, its block id is in
 * [0, num_blocks), and no two rows of one call target the same slot.  Rows
 * breaking the first two are skipped (never written out of bounds).
 */
int32_t pkv_kv_append(uint16_t* k_pool, uint16_t* v_pool,
                      const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* cu_new_lens, const int32_t* ctx_lens,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      int32_t num_seqs, int32_t total_new_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      void* stream);

/*
 * Bytes of device workspace pkv_paged_gqa_decode needs.  total_kv_tokens is a
 * host-side upper bound on the sum of seq_lens (<= 0: num_seqs * max_seq_len
 * is assumed).  Returns 0 for unsupported shapes.  The workspace must be
 * zero-filled once (or reset with pkv_decode_workspace_reset), before the
 * first decode call that uses it.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int64_t total_kv_tokens);

/*
 * Zero the chunk counters at the start of a decode workspace (its first
 * 16 KiB, the region every decode plan, bf16 or INT8, reserves for them).
 * A workspace must hold zero counters when a decode call starts; every
 * completed call leaves them so.  Use this on a workspace that was never
 * zero-filled, or whose last call did not complete (an aborted stream, a
 * launch that failed part-way): partials of such a call may otherwise be
 * merged wrongly by the next one.  Enqueued on `stream` as a kernel (no
 * memset node), so it may be captured in a graph.  Needs workspace_bytes >=
 * 16 KiB (every decode workspace is larger); errors: PKV_ERR_NULL_POINTER,
 * PKV_ERR_MISALIGNED (16-byte alignment), PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 */
int32_t pkv_decode_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_gqa_decode: one query row per sequence attends to all seq_lens[s]
 * keys of that sequence ("扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.2:
 * each group of consecutive query heads reads its KV head once).
 *
 *   out              [num_seqs][num_q_heads][head_dim] bf16, written
 *   q                [num_seqs][num_q_heads][head_dim] bf16
 *   k_pool, v_pool   as for kv_append (read only)
 *   block_table      [num_seqs][max_blocks_per_seq]
 *   seq_lens         [num_seqs] keys per sequence (the new token included),
 *                    each <= max_seq_len <= max_blocks_per_seq * block_size
 *   total_kv_tokens  host-side upper bound on sum(seq_lens) (<= 0: unknown,
 *                    num_seqs * max_seq_len is assumed); it sizes the splits
 *   scale            softmax scale (usually 1/sqrt(head_dim))
 *   workspace        device scratch of workspace_bytes >=
 *                    pkv_decode_workspace_bytes(...) with the same shapes and
 *                    total_kv_tokens, zero-filled before its first use (its
 *                    first 16 KiB hold per-(sequence, KV head) chunk counters,
 *                    which every completed call leaves at zero, whatever the
 *                    shapes); calls that share it must be ordered (same stream
 *                    or synchronised)
 *
 * Long sequences are split into chunks of keys whose partial results are
 * merged with a log-sum-exp combine: by the last of a sequence's chunks to
 * finish (counted in the workspace) when the launch is small, else by a
 * second kernel.  A sequence with seq_len 0 yields zeros.  Supports
 * num_seqs <= 8192.
 */
int32_t pkv_paged_gqa_decode(uint16_t* out, const uint16_t* q,
                             const uint16_t* k_pool, const uint16_t* v_pool,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * paged_gqa_decode_append: one decode step in one launch -- kv_append of one
 * new K/V row per sequence followed by paged_gqa_decode (the same two steps
 * the engine of "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" sections 4.3.1 and
 * 4.4.2 runs per generated token).
 *
 *   k_new, v_new     [num_seqs][num_kv_heads][head_dim] bf16: the row of
 *                    position seq_lens[s] - 1 of each sequence (a sequence
 *                    with seq_lens[s] == 0 appends nothing and yields zeros)
 *   k_pool, v_pool   written at that position (bit copies, as kv_append)
 *   other arguments  as for pkv_paged_gqa_decode (same workspace size)
 *
 * The outputs equal pkv_kv_append followed by pkv_paged_gqa_decode up to
 * summation order.  Preconditions as for both: the new rows' slots belong to
 * their sequence alone (no other sequence's table maps that slot).
 */
int32_t pkv_paged_gqa_decode_append(uint16_t* out, const uint16_t* q,
                                    const uint16_t* k_new, const uint16_t* v_new,
                                    uint16_t* k_pool, uint16_t* v_pool,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    float scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * paged_gqa_decode_append_static: pkv_paged_gqa_decode_append without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same kernels run on the library's own scratch: a static 32 MiB array
 * on each GPU the library is used on, held until the process ends.  Nothing
 * is allocated or freed, here or by the caller's runtime.
 *
 *   arguments        as for pkv_paged_gqa_decode_append, minus workspace
 *
 * Returns PKV_ERR_SCRATCH_LIMIT, launching nothing, when the call's plan
 * needs more than 32 MiB (pkv_decode_workspace_bytes(...) > 32 MiB: e.g.
 * more than about 1900 (sequence, split) partials at 32 query heads and
 * head_dim 128); other errors as for pkv_paged_gqa_decode_append.  The first
 * call on a device zeroes the scratch's chunk counters with a kernel on
 * `stream`.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's contents: calls that overlap on one GPU (different streams,
 * or host threads without ordering) race and must not be issued; calls on
 * one stream are ordered and safe.  A call that does not complete leaves the
 * scratch's counters undefined for the rest of the process.
 */
int32_t pkv_paged_gqa_decode_append_static(uint16_t* out, const uint16_t* q,
                                           const uint16_t* k_new, const uint16_t* v_new,
                                           uint16_t* k_pool, uint16_t* v_pool,
                                           const int32_t* block_table, int32_t max_blocks_per_seq,
                                           const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                           float scale, void* stream);

/*
 * paged_gqa_prefill: causal attention for a chunk of q_len_s query rows per
 * sequence ("扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.1: tiled,
 * without the full score matrix, skipping key tiles after the query tile).
 * Row r of sequence s sits at position seq_lens[s] - q_len_s + r and attends
 * to keys 0 .. that position (the chunk's own K/V must already be appended).
 *
 *   out              [total_q_tokens][num_q_heads][head_dim] bf16, written
 *   q                [total_q_tokens][num_q_heads][head_dim] bf16, rows packed
 *   cu_q_lens        [num_seqs + 1], q_len_s = cu_q_lens[s+1] - cu_q_lens[s],
 *                    each <= max_q_len and <= seq_lens[s]
 *   seq_lens         [num_seqs] cached + chunk tokens, each <= max_seq_len
 *                    <= max_blocks_per_seq * block_size
 */
int32_t pkv_paged_gqa_prefill(uint16_t* out, const uint16_t* q,
                              const int32_t* cu_q_lens, int32_t total_q_tokens, int32_t max_q_len,
                              const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t max_seq_len,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
