// C ABI of libpkv.so: argument validation, then the launches.  Nothing here
// touches device memory or synchronises; a rejected call launches nothing.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/pkv.h"
#include "../../include/pkv_blocks.h"
#include "../../include/pkv_int8.h"
#include "../../include/pkv_qkv.h"
#include "pkv_launch.h"

namespace pkv {

int device_cu_count() {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

namespace {

constexpr int32_t kMaxDecodeSeqs = 8192;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_in(int32_t x, int32_t lo, int32_t hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

// Shape rules shared by the attention calls.
int32_t check_heads(int32_t hq, int32_t hkv, int32_t d, int32_t bs) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return PKV_ERR_BAD_SHAPE;
    const int32_t g = hq / hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8) return PKV_ERR_BAD_SHAPE;
    if (d != 64 && d != 128) return PKV_ERR_BAD_SHAPE;
    if (!pow2_in(bs, 16, 256)) return PKV_ERR_BAD_SHAPE;
    return PKV_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int32_t status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL_POINTER: return "a required pointer is NULL";
        case PKV_ERR_BAD_SHAPE: return "sizes negative, inconsistent or unsupported";
        case PKV_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
        case PKV_ERR_WORKSPACE: return "decode workspace missing or too small";
        case PKV_ERR_HIP: return "a kernel launch failed";
        case PKV_ERR_NO_BLOCKS: return "not enough free or evictable KV blocks";
        case PKV_ERR_UNKNOWN_SEQ: return "no sequence with that id";
        case PKV_ERR_SCRATCH_LIMIT: return "the call needs more decode scratch than the library's static 32 MiB";
        default: return "unknown status";
    }
}

int32_t pkv_kv_append(uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* cu_new_lens, const int32_t* ctx_lens, const int32_t* block_table,
                      int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_new_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream) {
    if (num_seqs < 0 || total_new_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0)
        return PKV_ERR_BAD_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_BAD_SHAPE;
    if (!pow2_in(block_size, 16, 256)) return PKV_ERR_BAD_SHAPE;
    if (total_new_tokens > 0 && (num_seqs == 0 || num_blocks == 0 || max_blocks_per_seq == 0))
        return PKV_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
    if (total_new_tokens == 0) return PKV_OK;
    if (!k_pool || !v_pool || !k_new || !v_new || !cu_new_lens || !ctx_lens || !block_table)
        return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
        return PKV_ERR_MISALIGNED;
    AppendArgs a{k_pool, v_pool, k_new, v_new, cu_new_lens, ctx_lens, block_table, max_blocks_per_seq,
                 num_seqs, total_new_tokens, num_kv_heads, head_dim, block_size, num_blocks};
    return hip_status(launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

int32_t pkv_kv_append_int8(int8_t* k_codes, int8_t* v_codes, float* k_scales, float* v_scales, const uint16_t* k_new,
                           const uint16_t* v_new, const int32_t* cu_new_lens, const int32_t* ctx_lens,
                           const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_seqs,
                           int32_t total_new_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, void* stream) {
    if (num_seqs < 0 || total_new_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0)
        return PKV_ERR_BAD_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_BAD_SHAPE;
    if (!pow2_in(block_size, 32, 256)) return PKV_ERR_BAD_SHAPE;
    if (total_new_tokens > 0 && (num_seqs == 0 || num_blocks == 0 || max_blocks_per_seq == 0))
        return PKV_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
    if (total_new_tokens == 0) return PKV_OK;
    if (!k_codes || !v_codes || !k_scales || !v_scales || !k_new || !v_new || !cu_new_lens || !ctx_lens ||
        !block_table)
        return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) || !aligned16(v_scales) ||
        !aligned16(k_new) || !aligned16(v_new))
        return PKV_ERR_MISALIGNED;
    AppendArgs a{nullptr, nullptr, k_new, v_new, cu_new_lens, ctx_lens, block_table, max_blocks_per_seq,
                 num_seqs, total_new_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                 k_codes, v_codes, k_scales, v_scales};
    return hip_status(launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

int32_t pkv_qkv_project_append(uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool, const uint16_t* x,
                               const uint16_t* w_qkv, const int32_t* cu_new_lens, const int32_t* ctx_lens,
                               const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_seqs,
                               int32_t total_new_tokens, int32_t d_model, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream) {
    int32_t st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || total_new_tokens < 0 || num_blocks < 0 || max_blocks_per_seq < 0) return PKV_ERR_BAD_SHAPE;
    if (d_model <= 0 || d_model % 64 != 0) return PKV_ERR_BAD_SHAPE;
    if (total_new_tokens > 0 && (num_seqs == 0 || num_blocks == 0 || max_blocks_per_seq == 0))
        return PKV_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_ERR_BAD_SHAPE;
    const int64_t n_out = (int64_t)(num_q_heads + 2 * num_kv_heads) * head_dim;
    if ((int64_t)total_new_tokens * d_model >= (1ll << 30) || n_out * d_model >= (1ll << 30)) return PKV_ERR_BAD_SHAPE;
    if (total_new_tokens == 0) return PKV_OK;
    if (!q_out || !k_pool || !v_pool || !x || !w_qkv || !cu_new_lens || !ctx_lens || !block_table)
        return PKV_ERR_NULL_POINTER;
    if (!aligned16(q_out) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(x) || !aligned16(w_qkv))
        return PKV_ERR_MISALIGNED;
    QkvArgs a{q_out, k_pool, v_pool, x, w_qkv, cu_new_lens, ctx_lens, block_table, max_blocks_per_seq,
              num_seqs, total_new_tokens, d_model, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks};
    return hip_status(launch_qkv_append(a, static_cast<hipStream_t>(stream)));
}

int32_t pkv_copy_blocks(uint16_t* k_pool, uint16_t* v_pool, const int32_t* src_ids, const int32_t* dst_ids,
                        int32_t n_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, void* stream) {
    if (n_pairs < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_ERR_BAD_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_BAD_SHAPE;
    if (!pow2_in(block_size, 16, 256)) return PKV_ERR_BAD_SHAPE;
    if (n_pairs == 0) return PKV_OK;
    if (!k_pool || !v_pool || !src_ids || !dst_ids) return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_MISALIGNED;
    for (int32_t i = 0; i < n_pairs; ++i) {
        if (src_ids[i] < 0 || src_ids[i] >= num_blocks || dst_ids[i] < 0 || dst_ids[i] >= num_blocks)
            return PKV_ERR_BAD_SHAPE;
        for (int32_t j = 0; j < n_pairs; ++j)
            if (dst_ids[i] == src_ids[j] || (j != i && dst_ids[i] == dst_ids[j])) return PKV_ERR_BAD_SHAPE;
    }
    CopyBlocksArgs a{};
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.slab_elems = (int64_t)num_kv_heads * block_size * head_dim;
    for (int32_t i0 = 0; i0 < n_pairs; i0 += kCopyPairsPerLaunch) {
        a.n_pairs = n_pairs - i0 < kCopyPairsPerLaunch ? n_pairs - i0 : kCopyPairsPerLaunch;
        for (int32_t i = 0; i < a.n_pairs; ++i) {
            a.src[i] = src_ids[i0 + i];
            a.dst[i] = dst_ids[i0 + i];
        }
        const int32_t st = hip_status(launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
        if (st != PKV_OK) return st;
    }
    return PKV_OK;
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len, int64_t total_kv_tokens) {
    if (num_seqs < 0 || num_seqs > kMaxDecodeSeqs || max_seq_len < 0) return 0;
    if (check_heads(num_q_heads, num_kv_heads, head_dim, 16) != PKV_OK) return 0;
    return plan_decode_bf16(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, total_kv_tokens).bytes;
}

int32_t pkv_decode_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) return PKV_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return PKV_ERR_MISALIGNED;
    if (workspace_bytes < kCounterBytes) return PKV_ERR_WORKSPACE;
    return hip_status(launch_workspace_reset(workspace, static_cast<hipStream_t>(stream)));
}

size_t pkv_decode_int8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_seq_len, int64_t total_kv_tokens) {
    if (num_seqs < 0 || num_seqs > kMaxDecodeSeqs || max_seq_len < 0) return 0;
    if (check_heads(num_q_heads, num_kv_heads, head_dim, 32) != PKV_OK) return 0;
    return plan_decode_int8(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, total_kv_tokens).bytes;
}

}  // extern "C"

namespace {

// Validation shared by the decode entry points; on PKV_OK, `a` and `pl`
// describe the launch (nothing to launch when num_seqs == 0).  k / v are the
// cache arrays of the call (bf16 pools or INT8 codes); tile_keys picks the plan.
int32_t check_decode(DecodeArgs& a, DecodePlan& pl, const void* k, const void* v, int32_t tile_keys) {
    int32_t st = check_heads(a.num_q_heads, a.num_kv_heads, a.head_dim, a.block_size);
    if (st != PKV_OK) return st;
    if (a.num_seqs < 0 || a.num_seqs > kMaxDecodeSeqs || a.max_seq_len < 0 || a.num_blocks < 0 ||
        a.max_blocks_per_seq < 0)
        return PKV_ERR_BAD_SHAPE;
    if ((int64_t)a.max_seq_len > (int64_t)a.max_blocks_per_seq * a.block_size) return PKV_ERR_BAD_SHAPE;
    if (a.num_seqs == 0) return PKV_OK;
    if (!a.out || !a.q || !a.block_table || !a.seq_lens) return PKV_ERR_NULL_POINTER;
    if (a.max_seq_len > 0 && (!k || !v)) return PKV_ERR_NULL_POINTER;
    if (!aligned16(a.out) || !aligned16(a.q) || !aligned16(k) || !aligned16(v) || !aligned16(a.workspace))
        return PKV_ERR_MISALIGNED;
    pl = tile_keys == kDecodeInt8TileKeys
             ? plan_decode_int8(a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim, a.max_seq_len,
                                a.total_kv_tokens)
             : plan_decode_bf16(a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim, a.max_seq_len,
                                a.total_kv_tokens);
    if (!a.workspace || a.workspace_bytes < pl.bytes) return PKV_ERR_WORKSPACE;
    if (a.total_kv_tokens <= 0) a.total_kv_tokens = (int64_t)a.num_seqs * a.max_seq_len;
    return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_paged_gqa_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                             const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t max_seq_len, int64_t total_kv_tokens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float scale, void* workspace, size_t workspace_bytes, void* stream) {
    DecodeArgs a{out, q, k_pool, v_pool, block_table, max_blocks_per_seq, seq_lens, max_seq_len, total_kv_tokens,
                 num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                 workspace_bytes};
    DecodePlan pl{};
    const int32_t st = check_decode(a, pl, k_pool, v_pool, kDecodeTileKeys);
    if (st != PKV_OK || num_seqs == 0) return st;
    return hip_status(launch_decode(a, pl, static_cast<hipStream_t>(stream)));
}

int32_t pkv_paged_gqa_decode_append(uint16_t* out, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                    uint16_t* k_pool, uint16_t* v_pool, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                    int64_t total_kv_tokens, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    float scale, void* workspace, size_t workspace_bytes, void* stream) {
    DecodeArgs a{out, q, k_pool, v_pool, block_table, max_blocks_per_seq, seq_lens, max_seq_len, total_kv_tokens,
                 num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                 workspace_bytes, k_new, v_new, k_pool, v_pool};
    DecodePlan pl{};
    const int32_t st = check_decode(a, pl, k_pool, v_pool, kDecodeTileKeys);
    if (st != PKV_OK || num_seqs == 0) return st;
    if (!k_new || !v_new) return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_MISALIGNED;
    return hip_status(launch_decode(a, pl, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The decode scratch of pkv_paged_gqa_decode_append_static: one array per
// GPU the library runs on (each holds its own copy), kept until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: its device address comes from hipGetSymbolAddress, once per device,
// and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
std::vector<void*> scratch_ptr;  // per device: the device address of `scratch`

// The current device's scratch address; on the first call on a device its
// chunk counters are zeroed by a kernel on `stream` (before anything else
// that stream runs on the scratch).
int32_t device_scratch(void** ptr, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PKV_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if ((int)scratch_ptr.size() <= dev) scratch_ptr.resize(dev + 1, nullptr);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
        if (launch_workspace_reset(p, stream) != hipSuccess) return PKV_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_paged_gqa_decode_append_static(uint16_t* out, const uint16_t* q, const uint16_t* k_new,
                                           const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
                                           const int32_t* block_table, int32_t max_blocks_per_seq,
                                           const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                           void* stream) {
    // validate everything with a stand-in address (aligned, never touched) so
    // that a rejected call launches nothing, not even the first-call clear
    void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
    DecodeArgs a{out, q, k_pool, v_pool, block_table, max_blocks_per_seq, seq_lens, max_seq_len, total_kv_tokens,
                 num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, stand_in,
                 kScratchBytes, k_new, v_new, k_pool, v_pool};
    DecodePlan pl{};
    const int32_t st = check_decode(a, pl, k_pool, v_pool, kDecodeTileKeys);
    if (st == PKV_ERR_WORKSPACE) return PKV_ERR_SCRATCH_LIMIT;
    if (st != PKV_OK || num_seqs == 0) return st;
    if (!k_new || !v_new) return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_MISALIGNED;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t sst = device_scratch(&a.workspace, s);
    if (sst != PKV_OK) return sst;
    return hip_status(launch_decode(a, pl, s));
}

int32_t pkv_paged_gqa_decode_int8(uint16_t* out, const uint16_t* q, const int8_t* k_codes, const int8_t* v_codes,
                                  const float* k_scales, const float* v_scales, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                  int64_t total_kv_tokens, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  float scale, void* workspace, size_t workspace_bytes, void* stream) {
    if (block_size < 32) return PKV_ERR_BAD_SHAPE;  // a 32-key tile lies in one block
    DecodeArgs a{out, q, nullptr, nullptr, block_table, max_blocks_per_seq, seq_lens, max_seq_len, total_kv_tokens,
                 num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                 workspace_bytes, nullptr, nullptr, nullptr, nullptr, k_codes, v_codes, k_scales, v_scales};
    DecodePlan pl{};
    const int32_t st = check_decode(a, pl, k_codes, v_codes, kDecodeInt8TileKeys);
    if (st != PKV_OK || num_seqs == 0) return st;
    if (max_seq_len > 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_scales) || !aligned16(v_scales)) return PKV_ERR_MISALIGNED;
    return hip_status(launch_decode_int8(a, pl, static_cast<hipStream_t>(stream)));
}

int32_t pkv_paged_gqa_decode_append_int8(uint16_t* out, const uint16_t* q, const uint16_t* k_new,
                                         const uint16_t* v_new, int8_t* k_codes, int8_t* v_codes, float* k_scales,
                                         float* v_scales, const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, int64_t total_kv_tokens,
                                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    if (block_size < 32) return PKV_ERR_BAD_SHAPE;  // a 32-key tile lies in one block
    DecodeArgs a{out, q, nullptr, nullptr, block_table, max_blocks_per_seq, seq_lens, max_seq_len, total_kv_tokens,
                 num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                 workspace_bytes, k_new, v_new, nullptr, nullptr, k_codes, v_codes, k_scales, v_scales,
                 k_codes, v_codes, k_scales, v_scales};
    DecodePlan pl{};
    const int32_t st = check_decode(a, pl, k_codes, v_codes, kDecodeInt8TileKeys);
    if (st != PKV_OK || num_seqs == 0) return st;
    if (max_seq_len > 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL_POINTER;
    if (!k_new || !v_new) return PKV_ERR_NULL_POINTER;
    if (!aligned16(k_scales) || !aligned16(v_scales) || !aligned16(k_new) || !aligned16(v_new))
        return PKV_ERR_MISALIGNED;
    return hip_status(launch_decode_int8(a, pl, static_cast<hipStream_t>(stream)));
}

int32_t pkv_paged_gqa_prefill(uint16_t* out, const uint16_t* q, const int32_t* cu_q_lens, int32_t total_q_tokens,
                              int32_t max_q_len, const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t max_seq_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, void* stream) {
    int32_t st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
    if (st != PKV_OK) return st;
    if (num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0 || max_seq_len < 0 || num_blocks < 0 ||
        max_blocks_per_seq < 0)
        return PKV_ERR_BAD_SHAPE;
    if (max_q_len > max_seq_len || (int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
        return PKV_ERR_BAD_SHAPE;
    if (total_q_tokens > 0 && (num_seqs == 0 || max_q_len == 0)) return PKV_ERR_BAD_SHAPE;
    if ((int64_t)max_q_len * num_seqs < total_q_tokens) return PKV_ERR_BAD_SHAPE;
    if ((int64_t)((max_q_len + 127) / 128) * num_seqs * num_q_heads > INT32_MAX) return PKV_ERR_BAD_SHAPE;
    if (num_seqs == 0 || total_q_tokens == 0) return PKV_OK;
    if (!out || !q || !cu_q_lens || !k_pool || !v_pool || !block_table || !seq_lens) return PKV_ERR_NULL_POINTER;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_MISALIGNED;
    PrefillArgs a{out, q, cu_q_lens, total_q_tokens, max_q_len, k_pool, v_pool, block_table, max_blocks_per_seq,
                  seq_lens, max_seq_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                  scale};
    return hip_status(launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
