// kv_append: scatter new K/V rows into the paged pools.
//
// The paged cache of "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.3.1 keeps
// fixed-size blocks and fills a sequence's blocks in order, so logical position
// pos of sequence s is slot pos % B of block block_table[s][pos / B].  The copy
// is a pure bit move and HBM-bound: every thread moves one 16-byte piece (8 bf16)
// of K and the same piece of V, so a wave moves whole contiguous rows with
// 16-byte accesses on both sides.  Rows are read and written with the
// non-temporal hint (each byte is touched once; measured on 8130 prompt rows:
// 16.9 -> 14.6 us).  The INT8 append keeps plain accesses: its 8-byte code
// stores with the hint took 22.4 us against 20.3 us.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;

// Sequence owning packed row t: the last s with cu[s] <= t.  The first guess
// assumes equal row counts per sequence (exact for a decode step or equal
// chunks) and costs one round trip; otherwise a binary search over the
// num_seqs + 1 prefix follows (lanes of a wave search for nearby rows, so the
// probes mostly share addresses and hit in cache).
__device__ __forceinline__ int owner_seq(const int32_t* __restrict__ cu, int num_seqs, int total, int t) {
    const int guess = (int)((int64_t)t * num_seqs / total);
    if (cu[guess] <= t && (guess + 1 == num_seqs || cu[guess + 1] > t)) return guess;
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a) {
    constexpr int kPieces = D / 8;  // 16-byte pieces per row
    const int64_t idx = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    const int64_t total = (int64_t)a.total_new_tokens * a.num_kv_heads * kPieces;
    if (idx >= total) return;
    const int piece = (int)(idx % kPieces);
    const int64_t row_head = idx / kPieces;
    const int g = (int)(row_head % a.num_kv_heads);
    const int t = (int)(row_head / a.num_kv_heads);

    // the row's data does not depend on where it goes: load it first
    const int64_t src = ((int64_t)t * a.num_kv_heads + g) * D + piece * 8;
    const u32x4 kv = load16_nt(a.k_new + src);
    const u32x4 vv = load16_nt(a.v_new + src);

    const int s = owner_seq(a.cu_new_lens, a.num_seqs, a.total_new_tokens, t);
    const int64_t pos = (int64_t)a.ctx_lens[s] + (t - a.cu_new_lens[s]);
    const int64_t lblock = pos / a.block_size;
    if (pos < 0 || lblock >= a.max_blocks_per_seq) return;  // precondition broken: skip
    const int blk = a.block_table[(int64_t)s * a.max_blocks_per_seq + lblock];
    if (blk < 0 || blk >= a.num_blocks) return;
    const int slot = (int)(pos & (a.block_size - 1));
    const int64_t dst = (((int64_t)blk * a.num_kv_heads + g) * a.block_size + slot) * D + piece * 8;
    store16_nt(a.k_pool + dst, kv);
    store16_nt(a.v_pool + dst, vv);
}

// kv_append into an INT8 cache ("从零搭建AI工程能力：手写KV Cache与动态批处理实战"
// section 3.2): the placement of kv_append_kernel, each (token, KV head) row
// quantised on the way in.  A thread holds one 16-byte piece (8 values) of K
// and of V; the D / 8 lanes of a row find its maximum with a butterfly.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void kv_append_int8_kernel(AppendArgs a) {
    constexpr int kPieces = D / 8;
    const int64_t idx = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    const int64_t total = (int64_t)a.total_new_tokens * a.num_kv_heads * kPieces;
    if (idx >= total) return;  // whole rows only: a row's lanes all stay or all leave
    const int piece = (int)(idx % kPieces);
    const int64_t row_head = idx / kPieces;
    const int g = (int)(row_head % a.num_kv_heads);
    const int t = (int)(row_head / a.num_kv_heads);

    const int64_t src = ((int64_t)t * a.num_kv_heads + g) * D + piece * 8;
    float k_scale, v_scale;
    const u32x2 kq = quantize_piece<kPieces>(load16(a.k_new + src), &k_scale);
    const u32x2 vq = quantize_piece<kPieces>(load16(a.v_new + src), &v_scale);

    const int s = owner_seq(a.cu_new_lens, a.num_seqs, a.total_new_tokens, t);
    const int64_t pos = (int64_t)a.ctx_lens[s] + (t - a.cu_new_lens[s]);
    const int64_t lblock = pos / a.block_size;
    if (pos < 0 || lblock >= a.max_blocks_per_seq) return;  // precondition broken: skip
    const int blk = a.block_table[(int64_t)s * a.max_blocks_per_seq + lblock];
    if (blk < 0 || blk >= a.num_blocks) return;
    const int slot = (int)(pos & (a.block_size - 1));
    const int64_t row = ((int64_t)blk * a.num_kv_heads + g) * a.block_size + slot;
    *reinterpret_cast<u32x2*>(a.k_codes + row * D + piece * 8) = kq;
    *reinterpret_cast<u32x2*>(a.v_codes + row * D + piece * 8) = vq;
    if (piece == 0) {
        a.k_scales[row] = k_scale;
        a.v_scales[row] = v_scale;
    }
}

// Copy-on-write: block src[p] -> dst[p] of both pools, one 16-byte piece per
// thread; blockIdx.y is the pair.
__global__ __launch_bounds__(kAppendThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
    const int p = blockIdx.y;
    const int64_t e = ((int64_t)blockIdx.x * kAppendThreads + threadIdx.x) * 8;
    if (p >= a.n_pairs || e >= a.slab_elems) return;
    const int64_t s = (int64_t)a.src[p] * a.slab_elems + e, d = (int64_t)a.dst[p] * a.slab_elems + e;
    store16(a.k_pool + d, load16(a.k_pool + s));
    store16(a.v_pool + d, load16(a.v_pool + s));
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
    if (a.n_pairs <= 0) return hipSuccess;
    const int64_t pieces = a.slab_elems / 8;
    const dim3 grid((unsigned)((pieces + kAppendThreads - 1) / kAppendThreads), (unsigned)a.n_pairs);
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kAppendThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.total_new_tokens * a.num_kv_heads * (a.head_dim / 8);
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + kAppendThreads - 1) / kAppendThreads;
    if (a.k_codes) {
        if (a.head_dim == 128)
            hipLaunchKernelGGL(kv_append_int8_kernel<128>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(kv_append_int8_kernel<64>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, a);
    } else if (a.head_dim == 128) {
        hipLaunchKernelGGL(kv_append_kernel<128>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(kv_append_kernel<64>, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace pkv
