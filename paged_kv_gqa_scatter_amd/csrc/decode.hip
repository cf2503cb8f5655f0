// paged_gqa_decode: one query row per sequence over a paged KV cache, with the
// query heads of a GQA group sharing every K/V row they read.
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.2 reads a KV head once and
// uses it for all heads_per_group query heads of its group; that is the whole
// point here, because decode is bound by HBM bandwidth ("从零搭建AI工程能力"
// section 3.3).  The design on gfx950:
//
//  * Work item = (sequence, KV head, split of `chunk` keys), one wavefront
//    each.  A persistent grid walks the items; each workgroup first derives
//    the per-sequence split counts from seq_lens into LDS (no host sync).
//  * Lane layout: D/8 lanes cover one key row with 16-byte loads, so a wave
//    load reads 64/(D/8) consecutive rows of one contiguous (block, head) tile:
//    fully coalesced, block-gathered through the table.  The K row is held in
//    registers and used for all G query heads of the group (bf16 dot2 with
//    fp32 accumulation), then reduced across its D/8 lanes with xor shuffles.
//  * Online softmax in the exp2 domain (scale * log2 e folded into the scores),
//    running max / sum per head; rows past the sequence end are excluded by a
//    select, never multiplied by zero (unwritten slots may hold NaN).
//  * Splits of a sequence write a normalised partial and its log-sum-exp; a
//    second kernel merges them (out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M)).
//    A sequence with a single split is written directly.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kDecodeThreads = 256;  // 4 waves, each an independent work item
constexpr int kDecodeLoads = 4;      // wave-wide row loads per K (and V) per iteration
constexpr int kTargetItems = 8192;   // aim for about this many (split, KV head) items

struct DecodeKernelArgs {
    DecodeArgs a;
    int32_t chunk;
    int32_t log2_block;
    int64_t max_partials;
    int32_t* prefix;  // [num_seqs + 1]
    float* lse;       // [max_partials][Hq]
    float* part;      // [max_partials][Hq][D]
    float qk_scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

__device__ __forceinline__ int num_splits(int L, int chunk) { return L > 0 ? (L + chunk - 1) / chunk : 0; }

// Exclusive prefix of split counts over all sequences into s_prefix[0..S];
// every thread of the (256-thread) block takes part.
__device__ void split_prefix(const DecodeKernelArgs& p, int32_t* s_prefix, int32_t* s_wave) {
    const int S = p.a.num_seqs;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;
    const int tid = threadIdx.x;
    const int per = (S + kDecodeThreads - 1) / kDecodeThreads;
    const int lo = min(S, tid * per), hi = min(S, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += num_splits(clamp_len(p.a.seq_lens[i], cap), p.chunk);
    // inclusive scan: within the wave, then across the 4 waves
    const int lane = tid & 63, wave = tid >> 6;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += s_wave[w];
    incl += wave_off;
    int run = incl - sum;
    for (int i = lo; i < hi; ++i) {
        s_prefix[i] = run;
        run += num_splits(clamp_len(p.a.seq_lens[i], cap), p.chunk);
    }
    if (tid == kDecodeThreads - 1) s_prefix[S] = incl;
    __syncthreads();
}

template <int D, int G>
__device__ __forceinline__ void decode_item(const DecodeKernelArgs& p, int s, int g, int c, int nsplit,
                                            int64_t pidx, int lane) {
    constexpr int kLanesPerKey = D / 8;
    constexpr int kKeysPerLoad = kWave / kLanesPerKey;
    constexpr int kKeysPerIter = kDecodeLoads * kKeysPerLoad;
    const DecodeArgs& a = p.a;
    const int kq = lane / kLanesPerKey;  // which row of a wave load
    const int dl = lane % kLanesPerKey;  // which 8 dims of that row
    const int B = 1 << p.log2_block;
    const int L = clamp_len(a.seq_lens[s], a.max_blocks_per_seq << p.log2_block);
    const int k0 = c * p.chunk;
    const int k1 = min(k0 + p.chunk, L);
    const int Hq = a.num_q_heads;
    const int64_t head_stride = (int64_t)B * D;  // elements of one (block, head) tile

    u32x4 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = load16(a.q + ((int64_t)s * Hq + g * G + h) * D + dl * 8);

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }
    const int32_t* table = a.block_table + (int64_t)s * a.max_blocks_per_seq;

    for (int base = k0; base < k1; base += kKeysPerIter) {
        u32x4 kr[kDecodeLoads], vr[kDecodeLoads];
        bool valid[kDecodeLoads];
#pragma unroll
        for (int u = 0; u < kDecodeLoads; ++u) {
            const int j = base + u * kKeysPerLoad + kq;
            int blk = j < k1 ? table[j >> p.log2_block] : -1;
            valid[u] = (unsigned)blk < (unsigned)a.num_blocks;
            blk = valid[u] ? blk : 0;  // masked lanes keep an in-bounds address
            const int64_t off = ((int64_t)blk * a.num_kv_heads + g) * head_stride + (int64_t)(j & (B - 1)) * D + dl * 8;
            const u32x4 zero = {0u, 0u, 0u, 0u};
            kr[u] = valid[u] ? load16(a.k_pool + off) : zero;
            vr[u] = valid[u] ? load16(a.v_pool + off) : zero;
        }
        float sc[kDecodeLoads][G];
#pragma unroll
        for (int u = 0; u < kDecodeLoads; ++u)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = dot2_bf16(qv[h][i], kr[u][i], acc);
                sc[u][h] = group_sum<kLanesPerKey>(acc);
            }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < kDecodeLoads; ++u) {
                sc[u][h] = valid[u] ? sc[u][h] * p.qk_scale_log2 : -INFINITY;
                mt = fmaxf(mt, sc[u][h]);
            }
#pragma unroll
            for (int off = kLanesPerKey; off < kWave; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, kWave));
            const float m_new = fmaxf(m[h], mt);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m[h] - m_new);
            float pu[kDecodeLoads];
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < kDecodeLoads; ++u) {
                pu[u] = valid[u] ? fast_exp2(sc[u][h] - m_new) : 0.f;
                psum += pu[u];
            }
            l[h] = l[h] * alpha + psum;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float acc = o[h][i] * alpha;
#pragma unroll
                for (int u = 0; u < kDecodeLoads; ++u) {
                    const uint32_t w = vr[u][i >> 1];
                    acc += pu[u] * ((i & 1) ? bf16_hi(w) : bf16_lo(w));
                }
                o[h][i] = acc;
            }
            m[h] = m_new;
        }
    }

    // sum the per-row partials over the rows of a wave load (same max everywhere)
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int off = kLanesPerKey; off < kWave; off <<= 1) {
            l[h] += __shfl_xor(l[h], off, kWave);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] += __shfl_xor(o[h][i], off, kWave);
        }
    }
    if (kq != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int qh = g * G + h;
        const float inv = 1.f / l[h];
        if (nsplit == 1) {
            u32x4 packed;
#pragma unroll
            for (int i = 0; i < 4; ++i) packed[i] = pack_bf16x2(o[h][2 * i] * inv, o[h][2 * i + 1] * inv);
            store16(a.out + ((int64_t)s * Hq + qh) * D + dl * 8, packed);
        } else if (pidx < p.max_partials) {
            float* dst = p.part + (pidx * Hq + qh) * D + dl * 8;
            f32x4 lo4 = {o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv};
            f32x4 hi4 = {o[h][4] * inv, o[h][5] * inv, o[h][6] * inv, o[h][7] * inv};
            *reinterpret_cast<f32x4*>(dst) = lo4;
            *reinterpret_cast<f32x4*>(dst + 4) = hi4;
            if (dl == 0) p.lse[pidx * Hq + qh] = m[h] + log2f(l[h]);
        }
    }
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(DecodeKernelArgs p) {
    extern __shared__ int32_t s_prefix[];  // num_seqs + 1
    __shared__ int32_t s_wave[kDecodeThreads / kWave];
    split_prefix(p, s_prefix, s_wave);
    const int S = p.a.num_seqs;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i <= S; i += kDecodeThreads) p.prefix[i] = s_prefix[i];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Hkv = p.a.num_kv_heads;
    const int64_t total_items = (int64_t)s_prefix[S] * Hkv;
    const int64_t stride = (int64_t)gridDim.x * (kDecodeThreads / kWave);
    for (int64_t item = (int64_t)blockIdx.x * (kDecodeThreads / kWave) + wave; item < total_items; item += stride) {
        const int split = (int)(item / Hkv);
        const int g = (int)(item - (int64_t)split * Hkv);
        // the sequence owning this split: last s with s_prefix[s] <= split
        int lo = 0, hi = S - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_prefix[mid] <= split) lo = mid; else hi = mid - 1;
        }
        const int nsplit = s_prefix[lo + 1] - s_prefix[lo];
        decode_item<D, G>(p, lo, g, split - s_prefix[lo], nsplit, split, lane);
    }
}

// One thread per (sequence, query head, dim): merge the splits of a sequence.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeKernelArgs p) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int Hq = p.a.num_q_heads;
    const int d = (int)(idx % D);
    const int64_t sh = idx / D;
    const int h = (int)(sh % Hq);
    const int s = (int)(sh / Hq);
    if (s >= p.a.num_seqs) return;
    const int base = p.prefix[s];
    const int n = p.prefix[s + 1] - base;
    uint16_t* dst = p.a.out + ((int64_t)s * Hq + h) * D + d;
    if (n == 0) {  // no keys at all: the row is zero
        *dst = 0;
        return;
    }
    if (n == 1 || (int64_t)base + n > p.max_partials) return;
    float mx = -INFINITY;
    for (int i = 0; i < n; ++i) mx = fmaxf(mx, p.lse[(int64_t)(base + i) * Hq + h]);
    float num = 0.f, den = 0.f;
    for (int i = 0; i < n; ++i) {
        const float w = fast_exp2(p.lse[(int64_t)(base + i) * Hq + h] - mx);
        den += w;
        num += w * p.part[((int64_t)(base + i) * Hq + h) * D + d];
    }
    const __bf16 r = (__bf16)(num / den);
    *dst = __builtin_bit_cast(uint16_t, r);
}

template <int D, int G>
hipError_t launch_typed(const DecodeKernelArgs& kp, hipStream_t stream) {
    const DecodeArgs& a = kp.a;
    const size_t lds = sizeof(int32_t) * (size_t)(a.num_seqs + 1);
    // persistent grid: as many workgroups as can be resident, but no more than the work
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, G>, kDecodeThreads, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    const int64_t max_splits = (int64_t)a.num_seqs * ((a.max_seq_len + kp.chunk - 1) / kp.chunk);
    const int64_t items = (max_splits < kp.max_partials ? max_splits : kp.max_partials) * a.num_kv_heads;
    int64_t blocks = (items + 3) / 4;
    const int64_t resident = (int64_t)per_cu * device_cu_count();
    if (blocks > resident) blocks = resident;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3((unsigned)blocks), dim3(kDecodeThreads), lds, stream, kp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)a.num_seqs * a.num_q_heads * D;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, kp);
    return hipGetLastError();
}

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

}  // namespace

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_seq_len, int64_t total_kv_tokens) {
    DecodePlan pl{};
    const int64_t bound_tokens = (int64_t)num_seqs * max_seq_len;
    int64_t total = total_kv_tokens > 0 ? total_kv_tokens : bound_tokens;
    if (total > bound_tokens) total = bound_tokens;
    const int64_t key_heads = total * num_kv_heads;
    int chunk = 64;
    while (chunk < 2048 && (int64_t)chunk * 2 * kTargetItems <= key_heads) chunk *= 2;
    pl.chunk = chunk;
    const int64_t by_len = (int64_t)num_seqs * ((max_seq_len + chunk - 1) / chunk);
    const int64_t by_total = (total + chunk - 1) / chunk + num_seqs;
    pl.max_partials = by_len < by_total ? by_len : by_total;
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    pl.prefix_offset = 0;
    pl.lse_offset = align(sizeof(int32_t) * (size_t)(num_seqs + 1));
    pl.o_offset = align(pl.lse_offset + sizeof(float) * (size_t)pl.max_partials * num_q_heads);
    pl.bytes = pl.o_offset + sizeof(float) * (size_t)pl.max_partials * num_q_heads * head_dim;
    return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    DecodeKernelArgs kp;
    kp.a = a;
    kp.chunk = pl.chunk;
    kp.log2_block = ilog2(a.block_size);
    kp.max_partials = pl.max_partials;
    char* ws = static_cast<char*>(a.workspace);
    kp.prefix = reinterpret_cast<int32_t*>(ws + pl.prefix_offset);
    kp.lse = reinterpret_cast<float*>(ws + pl.lse_offset);
    kp.part = reinterpret_cast<float*>(ws + pl.o_offset);
    kp.qk_scale_log2 = a.scale * kLog2e;
    const int G = a.num_q_heads / a.num_kv_heads;
    if (a.head_dim == 128) {
        switch (G) {
            case 1: return launch_typed<128, 1>(kp, stream);
            case 2: return launch_typed<128, 2>(kp, stream);
            case 4: return launch_typed<128, 4>(kp, stream);
            default: return launch_typed<128, 8>(kp, stream);
        }
    }
    switch (G) {
        case 1: return launch_typed<64, 1>(kp, stream);
        case 2: return launch_typed<64, 2>(kp, stream);
        case 4: return launch_typed<64, 4>(kp, stream);
        default: return launch_typed<64, 8>(kp, stream);
    }
}

}  // namespace pkv
