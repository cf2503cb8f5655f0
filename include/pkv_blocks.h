/*
 * pkv_blocks.h - host-side paged KV block manager and prefix cache for libpkv.
 *
 * The paged cache of "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.3.1 cuts
 * the KV cache into fixed-size blocks taken from a free pool in O(1), each
 * sequence keeping its own list of blocks and opening a new one when its last
 * block is full; section 4.4.4 reuses the KV of a prefix that an earlier
 * request already computed, matched by a hash of its token ids (the whole
 * prompt first, then ever shorter prefixes).  This manager does that
 * bookkeeping for the physical block ids [0, num_blocks) of the device pools
 * the kernels of pkv.h read and write; it never touches device memory.  Its
 * block tables are the block_table arguments of those kernels.
 *
 * Sharing and copy-on-write: a block may be held by several sequences (a
 * shared prefix) and by the prefix cache, with a reference count.  A block's
 * fill level is the number of its slots that hold K/V.  A sequence appends in
 * place only into its own frontier (its length within the block equals the
 * block's fill level and no other holder can write there); otherwise the
 * block is first replaced by a private copy, and the caller copies the K/V
 * slots on the device (pkv_copy_blocks) before writing the new rows.
 *
 * Cached prefixes are whole blocks plus, optionally, one partially filled
 * block at the end.  A block that only the cache holds stays cached until an
 * allocation finds the free pool empty; then the least recently used cached
 * prefix end (a block no longer prefix is built on) is evicted.
 *
 * Not thread-safe: one manager per scheduler thread, or external locking.
 * Status codes are those of pkv.h plus PKV_ERR_NO_BLOCKS / PKV_ERR_UNKNOWN_SEQ;
 * a call that fails changes nothing.
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PKV_ERR_NO_BLOCKS = 6,    /* not enough free or evictable blocks            */
    PKV_ERR_UNKNOWN_SEQ = 7   /* no sequence with that id                       */
};

typedef struct pkv_block_manager pkv_block_manager;

/* A manager of block ids [0, num_blocks) of block_size tokens each
 * (block_size a power of two in [16, 256]); NULL on bad sizes. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Blocks an allocation can obtain now: free ones plus cached ones that no
 * sequence holds. */
int32_t pkv_bm_available(const pkv_block_manager* bm);

/* Tokens of sequence seq_id, or -1 if there is no such sequence. */
int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id);

/*
 * Reserve positions len .. len + n_tokens - 1 of sequence seq_id (created
 * empty if unknown) and grow its block list: a new block whenever the last
 * one is full.  If the first new position falls in a block that the sequence
 * may not write in place (see above), that block is replaced by a fresh one
 * and *cow_src / *cow_dst receive the old and new ids: the caller must copy
 * the first len % block_size slots of every KV head from cow_src to cow_dst
 * (pkv_copy_blocks copies whole blocks, which also does) before the new rows
 * are written.  Otherwise both are set to -1.  cow_src / cow_dst may not be
 * NULL.  PKV_ERR_NO_BLOCKS if the blocks needed are not available.
 */
int32_t pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int32_t n_tokens, int32_t* cow_src,
                      int32_t* cow_dst);

/* Drop a sequence; its blocks return to the free pool unless another
 * sequence or the prefix cache still holds them. */
int32_t pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/*
 * Block tables of n sequences, row-major [n][max_blocks_per_seq] int32:
 * entry j of row i is the physical block of logical block j of seq_ids[i],
 * and -1 past its last block.  PKV_ERR_BAD_SHAPE if a sequence has more
 * blocks than max_blocks_per_seq (nothing written).
 */
int32_t pkv_bm_block_table(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                           int32_t max_blocks_per_seq, int32_t* table);

/*
 * Remember that the first n_tokens positions of sequence seq_id hold the
 * K/V of token ids tokens[0 .. n_tokens - 1] (n_tokens <= its length), so
 * that pkv_bm_fork can reuse them: every block they cover becomes findable
 * by content, and the cache holds a reference to it.
 */
int32_t pkv_bm_cache_prefix(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n_tokens);

/*
 * Start sequence new_seq_id (which must not exist) on the longest cached
 * prefix of tokens[0 .. n_tokens - 1]: *matched receives how many of those
 * tokens' K/V it shares (0: an empty sequence).  The caller then appends and
 * prefills positions *matched .. n_tokens - 1.
 */
int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t new_seq_id, const int32_t* tokens, int32_t n_tokens,
                    int32_t* matched);

/*
 * Device side of copy-on-write: copy whole blocks src_ids[i] -> dst_ids[i]
 * of both pools ([num_blocks][num_kv_heads][block_size][head_dim] bf16), for
 * i < n_pairs.  src_ids / dst_ids are HOST arrays (read before the call
 * returns); the copies are enqueued on `stream`.  Ids must be in
 * [0, num_blocks) and no dst may also be a src or repeat (PKV_ERR_BAD_SHAPE
 * otherwise, nothing launched).
 */
int32_t pkv_copy_blocks(uint16_t* k_pool, uint16_t* v_pool, const int32_t* src_ids, const int32_t* dst_ids,
                        int32_t n_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
