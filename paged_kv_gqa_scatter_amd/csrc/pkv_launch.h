// Host-side launch interface between the C ABI (pkv_api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct AppendArgs {
    uint16_t* k_pool;
    uint16_t* v_pool;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* cu_new_lens;
    const int32_t* ctx_lens;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    int32_t num_seqs;
    int32_t total_new_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    // INT8 cache (else null): codes [num_blocks][num_kv_heads][block_size][head_dim]
    // and one fp32 scale per slot [num_blocks][num_kv_heads][block_size];
    // k_pool / v_pool are then unused
    int8_t* k_codes;
    int8_t* v_codes;
    float* k_scales;
    float* v_scales;
};

struct DecodeArgs {
    uint16_t* out;
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    const int32_t* seq_lens;
    int32_t max_seq_len;
    int64_t total_kv_tokens;  // host bound on sum(seq_lens), > 0
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    float scale;
    void* workspace;
    size_t workspace_bytes;
    // decode_append only (else null): one new K/V row per sequence
    // [num_seqs][num_kv_heads][head_dim], at position seq_lens[s] - 1, and
    // the same pools, writable
    const uint16_t* k_new;
    const uint16_t* v_new;
    uint16_t* k_pool_w;
    uint16_t* v_pool_w;
    // INT8 cache (decode_int8 only): codes and per-slot scales as in AppendArgs
    const int8_t* k_codes;
    const int8_t* v_codes;
    const float* k_scales;
    const float* v_scales;
    // decode_append_int8 (with k_new / v_new): the same cache, writable
    int8_t* k_codes_w;
    int8_t* v_codes_w;
    float* k_scales_w;
    float* v_scales_w;
};

struct PrefillArgs {
    uint16_t* out;
    const uint16_t* q;
    const int32_t* cu_q_lens;
    int32_t total_q_tokens;
    int32_t max_q_len;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    const int32_t* seq_lens;
    int32_t max_seq_len;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    float scale;
};

// Fused QKV projection + paged append: y = x W^T, q part to q_out, k / v
// parts to the pools at each token's slot.
struct QkvArgs {
    uint16_t* q_out;        // [T][Hq * D]
    uint16_t* k_pool;
    uint16_t* v_pool;
    const uint16_t* x;      // [T][d_model]
    const uint16_t* w;      // [(Hq + 2 Hkv) * D][d_model]
    const int32_t* cu_new_lens;
    const int32_t* ctx_lens;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    int32_t num_seqs;
    int32_t total_new_tokens;
    int32_t d_model;        // a multiple of 64
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
};

// Decode split plan: keys per split and workspace layout, a pure function of
// host-known shapes so that the size query and the launch always agree.
// tile_keys: keys per tile of the kernel (kDecodeTileKeys / kDecodeInt8TileKeys).
constexpr int32_t kDecodeTileKeys = 16;
constexpr int32_t kDecodeInt8TileKeys = 32;
struct DecodePlan {
    int32_t ring;             // LDS stages per wave of the split kernel (2 or 4)
    int32_t chunk;            // keys per work item (a multiple of 16 tiles)
    int32_t max_chunks;       // chunks of the longest sequence
    int32_t persistent;       // 1: persistent grid over a compact item list
    int32_t pack;             // 1: decode sequences sharing a chunk together (bf16)
    int32_t fused;            // 1: the split kernel merges (counters), no merge kernel
    int32_t last_first;       // 1: a one-round direct grid deals its last chunks first
    int64_t items;            // bound on (chunk, KV head) work items
    int64_t max_partials;     // (sequence, split) slots the workspace holds
    size_t counter_offset;    // int32 [num_seqs][num_kv_heads] chunk counters (fused merge)
    size_t prefix_offset;     // int32 [num_seqs + 1] chunk prefix (persistent grid)
    size_t lse_offset;        // float [max_partials][num_q_heads]
    size_t o_offset;          // float [max_partials][num_q_heads][head_dim]
    size_t bytes;
};

// The split kernel merges a sequence's partials itself (the last of its
// chunks to finish, counted per (sequence, KV head)) when the grid is direct,
// no sequences are packed and the counters fit the fixed region at the start
// of every decode workspace; otherwise a merge kernel follows it.
constexpr int64_t kMaxFusedPairs = 4096;
constexpr size_t kCounterBytes = sizeof(int32_t) * kMaxFusedPairs;
inline int32_t can_fuse_merge(const DecodePlan& pl, int32_t num_seqs, int32_t num_kv_heads) {
    return !pl.persistent && !pl.pack && pl.max_chunks >= 2 && (int64_t)num_seqs * num_kv_heads <= kMaxFusedPairs;
}

// plan_decode: the split of a kernel whose tiles hold tile_keys keys and of
// which wgs_per_cu workgroups are resident on one CU; the plan of each cache
// format (which also picks its ring depth) comes from plan_decode_bf16 /
// plan_decode_int8.
// max_chunk_keys > 0 caps the keys per work item.
DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_seq_len, int64_t total_kv_tokens, int32_t tile_keys, int32_t wgs_per_cu,
                       int32_t max_chunk_keys = 0);
DecodePlan plan_decode_bf16(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_seq_len, int64_t total_kv_tokens);
DecodePlan plan_decode_int8(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_seq_len, int64_t total_kv_tokens);

// Whole-block copies of both pools (copy-on-write of a shared block).
constexpr int kCopyPairsPerLaunch = 32;
struct CopyBlocksArgs {
    uint16_t* k_pool;
    uint16_t* v_pool;
    int32_t src[kCopyPairsPerLaunch];
    int32_t dst[kCopyPairsPerLaunch];
    int32_t n_pairs;         // <= kCopyPairsPerLaunch
    int64_t slab_elems;      // num_kv_heads * block_size * head_dim
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);
// Zero the chunk counters at the start of a decode workspace (a kernel, so
// that the call may sit in a captured graph).
hipError_t launch_workspace_reset(void* workspace, hipStream_t stream);
hipError_t launch_decode_int8(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_qkv_append(const QkvArgs& a, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace pkv
