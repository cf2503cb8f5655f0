// paged_gqa_decode: one query row per sequence over a paged KV cache, with the
// query heads of a GQA group sharing every K/V row they read.
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.2 reads a KV head once and
// uses it for all heads_per_group query heads of its group; that is the whole
// point here, because decode is bound by HBM bandwidth ("从零搭建AI工程能力"
// section 3.3).  The design on gfx950:
//
//  * Work item = (sequence, KV head, chunk of `chunk` keys), one workgroup of
//    4 waves.  Each wave takes every 4th step of 64 keys of the chunk; the
//    waves' partial softmax states are merged through LDS.  Short batches use
//    a direct grid over (chunk, sequence, KV head) whose empty items exit at
//    once; long, uneven batches use a persistent grid over a compact item list
//    that each workgroup derives from seq_lens (a block scan in LDS).  Either
//    way nothing is read back to the host, and the KV head sits in the low
//    bits of the workgroup index, so items of one KV head run on one XCD
//    (workgroups are dealt round-robin over the 8 XCDs) and K/V rows shared
//    between sequences (a common prefix) are re-read from that XCD's L2.
//  * Within a step all K and V loads are issued before any is used: D/8 lanes
//    cover one row with 16-byte loads, a wave load reads 64/(D/8) consecutive
//    rows of one contiguous (block, head) tile, and D/8 such loads cover the 64
//    keys -- 32 KB in flight per wave.  Each K row, once in registers, serves
//    all G query heads of the group.
//  * Scores: each lane dots its 8 dims of each of its keys with the G query
//    heads (bf16 dot2, fp32 accumulate).  The D/8 partial sums are folded
//    across the row's lanes with DPP moves in a transposing order: at every
//    fold a lane keeps half of its values and adds its partner's copy of that
//    half, so after log2(D/8) folds each lane holds the complete G scores of
//    exactly one key.  The softmax then costs G exponentials per lane.
//  * Online softmax in the exp2 domain (scale * log2 e folded in); the step
//    max is a wave reduction; rows past the sequence end are excluded by a
//    select, never multiplied by zero (unwritten slots may hold NaN).
//  * P V: each lane needs the weights of the keys whose V rows it holds; they
//    are broadcast inside each group of D/8 lanes (DPP row broadcast or an LDS
//    swizzle) and accumulated into G x 8 fp32 outputs per lane.
//  * Chunks of a sequence write a normalised partial and its log2-sum-exp; a
//    second kernel merges them in one pass with a running maximum
//    (out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M)).  The hand-off goes
//    through a kernel boundary on purpose: the L2 is per XCD, so a device-scope
//    fence inside the kernel would write back and invalidate an XCD's whole
//    L2 under every other workgroup's streaming loads.  A sequence with one
//    chunk is written directly (and the merge kernel is not launched when no
//    sequence can have two); a sequence with no keys gets zeros.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kDecodeThreads = 256;  // 4 waves share one work item
constexpr int kDecodeWaves = kDecodeThreads / kWave;
constexpr int kStepKeys = 64;        // keys whose K/V loads are in flight together
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.f;  // log2 of the largest weight a stale running max may give

struct DecodeKernelArgs {
    DecodeArgs a;
    int32_t chunk;       // keys per work item (multiple of 4 * 64)
    int32_t log2_block;
    int32_t max_chunks;  // chunks of the longest sequence
    int32_t persistent;  // 1: persistent grid over the compact item list
    int64_t max_partials;
    float* lse;         // [max_partials][Hq]
    float* part;        // [max_partials][Hq][D]
    float qk_scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

__device__ __forceinline__ int num_chunks(int L, int chunk) { return L > 0 ? (L + chunk - 1) / chunk : 0; }

// Exclusive prefix of chunk counts over all sequences into s_prefix[0..S];
// every thread of the block takes part.
__device__ void chunk_prefix(const DecodeKernelArgs& p, int32_t* s_prefix, int32_t* s_wave) {
    const int S = p.a.num_seqs;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;
    const int tid = threadIdx.x;
    const int per = (S + kDecodeThreads - 1) / kDecodeThreads;
    const int lo = min(S, tid * per), hi = min(S, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += num_chunks(clamp_len(p.a.seq_lens[i], cap), p.chunk);
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
        run += num_chunks(clamp_len(p.a.seq_lens[i], cap), p.chunk);
    }
    if (tid == kDecodeThreads - 1) s_prefix[S] = incl;
    __syncthreads();
}

// One fold of the transposing reduction over the lanes of a key row: lanes
// whose `upper` bit is set keep the upper half of v[0..N) and the others the
// lower half; each adds its partner's copy of the half it keeps.  kCtrl must
// pair every lane with one whose `upper` bit differs and whose bits above it
// agree.
template <int N, int kCtrl>
__device__ __forceinline__ void fold(float* v, bool upper) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float keep = upper ? v[N / 2 + i] : v[i];
        const float send = upper ? v[i] : v[N / 2 + i];
        v[i] = keep + dpp<kCtrl>(send);
    }
}

// Reductions over the 64 lanes, returned wave-uniform: DPP inside each row of
// 16 lanes; then every lane of a row holds the row's result, and the row
// broadcasts 15 and 31 fold rows 0..2 into row 3, whose last lane is read into
// a scalar register.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    x = fmaxf(x, dpp<kDppHalfMirror>(x));
    x = fmaxf(x, dpp<kDppMirror>(x));
    x = fmaxf(x, dpp_rows<kDppRowBcast15, 0xA>(x, x));
    x = fmaxf(x, dpp_rows<kDppRowBcast31, 0xC>(x, x));
    return readlane(x, 63);
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppMirror>(x);
    x += dpp_rows<kDppRowBcast15, 0xA>(0.f, x);
    x += dpp_rows<kDppRowBcast31, 0xC>(0.f, x);
    return readlane(x, 63);
}

// Broadcast lane u of each group of kLanes lanes (16: DPP row broadcast;
// 8: LDS swizzle in broadcast mode).
template <int kLanes, int u>
__device__ __forceinline__ float group_bcast(float x) {
    if constexpr (kLanes == 16) {
        return dpp<kDppRowBcast0 + u>(x);
    } else {
        static_assert(kLanes == 8, "groups of 8 or 16 lanes");
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x18 | (u << 5)));
    }
}

// P V for the key pair (2a, 2a+1) of a step: their bf16 weights (already
// rounded, so the packing is exact) times their V rows, two keys per dot2.
template <int kLanes, int G, int a>
__device__ __forceinline__ void pv_pair(float (&o)[G][8], const float (&pk)[G], const u32x4& va, const u32x4& vb) {
    uint32_t pp[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        pp[h] = pack_bf16x2(group_bcast<kLanes, 2 * a>(pk[h]), group_bcast<kLanes, 2 * a + 1>(pk[h]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (va[i] & 0xFFFFu) | (vb[i] << 16);         // dim 2i of keys 2a, 2a+1
        const uint32_t hi = (va[i] >> 16) | (vb[i] & 0xFFFF0000u);     // dim 2i+1
#pragma unroll
        for (int h = 0; h < G; ++h) {
            o[h][2 * i] = dot2_bf16(lo, pp[h], o[h][2 * i]);
            o[h][2 * i + 1] = dot2_bf16(hi, pp[h], o[h][2 * i + 1]);
        }
    }
}

template <int kLanes, int G, int a>
struct PvAll {
    static __device__ __forceinline__ void run(float (&o)[G][8], const float (&pk)[G], const u32x4* vr) {
        PvAll<kLanes, G, a - 1>::run(o, pk, vr);
        pv_pair<kLanes, G, a - 1>(o, pk, vr[2 * a - 2], vr[2 * a - 1]);
    }
};
template <int kLanes, int G>
struct PvAll<kLanes, G, 0> {
    static __device__ __forceinline__ void run(float (&)[G][8], const float (&)[G], const u32x4*) {}
};

// LDS of one workgroup: the waves' softmax states, then the item's merge.
// o keeps each wave's per-row partial sums (rows of a wave load are summed by
// the merge, which is cheaper than cross-row lane exchanges).
template <int D, int G>
struct DecodeShared {
    static constexpr int kRows = kWave / (D / 8);  // keys per wave load
    float o[kDecodeWaves][kRows][G][D];
    float m[kDecodeWaves][G];
    float l[kDecodeWaves][G];
    int32_t wave_sum[kDecodeWaves];
};

// Steps base = k_begin + wave*64, + 4*64, ... below k_end of sequence s, KV
// head g; leaves the running max m (wave-uniform), the per-key-lane sums l and
// the per-row outputs o.  first_blk is the block id of this wave's first step,
// loaded by the caller together with the sequence length.
template <int D, int G, bool kWholeStep>
__device__ __forceinline__ void wave_steps(const DecodeKernelArgs& p, int s, int g, int k_begin, int k_end,
                                           int first_blk, const u32x4 (&qv)[G], int lane, int wave, float (&m)[G],
                                           float (&l)[G], float (&o)[G][8]) {
    constexpr int kLanesPerKey = D / 8;                 // lanes per key row (16 B each)
    constexpr int kKeysPerLoad = kWave / kLanesPerKey;  // rows per wave load
    constexpr int kLoads = kStepKeys / kKeysPerLoad;    // wave loads per step (= kLanesPerKey)
    static_assert(kLoads == kLanesPerKey, "one key per lane after the fold");
    const DecodeArgs& a = p.a;
    const int kq = lane / kLanesPerKey;
    const int dl = lane % kLanesPerKey;
    const int B = 1 << p.log2_block;
    const int64_t tile = (int64_t)B * D;  // elements of one (block, head) tile
    const int32_t* table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    const int last_entry = a.max_blocks_per_seq - 1;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    int blk_step = first_blk;  // the whole step's block when kWholeStep (blocks of >= 64 keys)

    for (int base = k_begin + wave * kStepKeys; base < k_end; base += kDecodeWaves * kStepKeys) {
        // ---- block ids of the step's rows first (one batch of loads when blocks
        //      are smaller than a step), so that the K/V loads below go out back
        //      to back with no wait between them
        int blks[kLoads];
        if constexpr (kWholeStep) {
#pragma unroll
            for (int u = 0; u < kLoads; ++u) blks[u] = blk_step;
        } else {
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int j = base + u * kKeysPerLoad + kq;
                blks[u] = table[min(j, k_end - 1) >> p.log2_block];
            }
        }
        // ---- issue every K and V load of the step
        u32x4 kr[kLoads], vr[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int j = base + u * kKeysPerLoad + kq;
            const bool ok = j < k_end && (unsigned)blks[u] < (unsigned)a.num_blocks;
            const int blk = ok ? blks[u] : 0;  // masked lanes keep an in-bounds address
            const int64_t off = ((int64_t)blk * a.num_kv_heads + g) * tile + (int64_t)(j & (B - 1)) * D + dl * 8;
            kr[u] = ok ? load16(a.k_pool + off) : zero;
            vr[u] = ok ? load16(a.v_pool + off) : zero;
        }
        const int cur_blk = blk_step;
        blk_step = table[min((base + kDecodeWaves * kStepKeys) >> p.log2_block, last_entry)];  // next step's
        // ---- partial dots: sc[u * G + h] over this lane's 8 dims
        float sc[kLoads * G];
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = dot2_bf16(qv[h][i], kr[u][i], acc);
                sc[u * G + h] = acc;
            }
        // ---- transposing fold: afterwards sc[0..G) are the scores of key u = dl
        if constexpr (kLanesPerKey == 16) {
            fold<16 * G, kDppMirror>(sc, dl & 8);
            fold<8 * G, kDppHalfMirror>(sc, dl & 4);
            fold<4 * G, kDppXor2>(sc, dl & 2);
            fold<2 * G, kDppXor1>(sc, dl & 1);
        } else {
            fold<8 * G, kDppHalfMirror>(sc, dl & 4);
            fold<4 * G, kDppXor2>(sc, dl & 2);
            fold<2 * G, kDppXor1>(sc, dl & 1);
        }
        const int key = base + dl * kKeysPerLoad + kq;
        bool valid = key < k_end;
        if (valid) valid = (unsigned)(kWholeStep ? cur_blk : table[key >> p.log2_block]) < (unsigned)a.num_blocks;
        // ---- online softmax (exp2 domain), one key per lane; the running max
        //      is wave-uniform and moves only when it would grow by > 2^8
        float pk[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float z = valid ? sc[h] * p.qk_scale_log2 : -INFINITY;
            const float mx = wave_max(z);
            if (mx > m[h] + kRescaleSlack) {
                const float alpha = fast_exp2(m[h] - mx);  // 0 while m is -inf
                l[h] *= alpha;
#pragma unroll
                for (int i = 0; i < 8; ++i) o[h][i] *= alpha;
                m[h] = mx;
            }
            // weights are rounded to bf16 for the dot2 P V; the sums take the same values
            pk[h] = valid ? round_bf16(fast_exp2(z - m[h])) : 0.f;
            l[h] += pk[h];
        }
        // ---- P V over the step's keys, two keys per dot2
        PvAll<kLanesPerKey, G, kLoads / 2>::run(o, pk, vr);
    }
}

// Merge kernel: one workgroup per (sequence, KV head) merges that sequence's
// chunk partials into the bf16 output, one pass with a running maximum so all
// loads are independent.  Sequences with fewer than two chunks were finished
// by the split kernel.
template <int D, int G>
constexpr int elems_per_thread() { return (G * D + kDecodeThreads - 1) / kDecodeThreads; }

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_merge_kernel(DecodeKernelArgs p, const int32_t* prefix) {
    constexpr int kElems = elems_per_thread<D, G>();  // outputs per thread
    const int Hkv = p.a.num_kv_heads, Hq = p.a.num_q_heads;
    const int g = blockIdx.x % Hkv, s = blockIdx.x / Hkv;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;
    const int n = num_chunks(clamp_len(p.a.seq_lens[s], cap), p.chunk);
    if (n < 2) return;
    const int64_t base = p.persistent ? (int64_t)prefix[s] : (int64_t)s * p.max_chunks;
    if (base + n > p.max_partials) return;  // precondition broken: no partials to merge
    const int e0 = threadIdx.x * kElems;
    if (e0 >= G * D) return;
    const int h = e0 / D, d0 = e0 % D;
    const int qh = g * G + h;
    float mx = -INFINITY, den = 0.f, num[kElems];
#pragma unroll
    for (int k = 0; k < kElems; ++k) num[k] = 0.f;
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        const float li = p.lse[(base + i) * Hq + qh];
        const float* src = p.part + ((base + i) * Hq + qh) * D + d0;
        const float m_new = fmaxf(mx, li);
        const float a_old = fast_exp2(mx - m_new);  // 0 on the first partial
        const float w = fast_exp2(li - m_new);
        den = den * a_old + w;
#pragma unroll
        for (int k = 0; k < kElems; ++k) num[k] = num[k] * a_old + w * src[k];
        mx = m_new;
    }
    const float inv = 1.f / den;
    uint16_t* dst = p.a.out + ((int64_t)s * Hq + qh) * D + d0;
#pragma unroll
    for (int k = 0; k < kElems; ++k) dst[k] = __builtin_bit_cast(uint16_t, (__bf16)(num[k] * inv));
}

// What a work item needs before its first K/V load, fetched in one round
// trip: the sequence length, the G query rows and this wave's first block id.
template <int D, int G>
struct ItemInputs {
    int L_raw;
    int first_blk;
    u32x4 qv[G];
};

template <int D, int G>
__device__ __forceinline__ ItemInputs<D, G> load_item_inputs(const DecodeKernelArgs& p, int s, int g, int c) {
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int dl = lane % (D / 8);
    ItemInputs<D, G> in;
    in.L_raw = a.seq_lens[s];
#pragma unroll
    for (int h = 0; h < G; ++h) in.qv[h] = load16(a.q + ((int64_t)s * a.num_q_heads + g * G + h) * D + dl * 8);
    in.first_blk = a.block_table[(int64_t)s * a.max_blocks_per_seq +
                                 min((c * p.chunk + wave * kStepKeys) >> p.log2_block, a.max_blocks_per_seq - 1)];
    return in;
}

// One work item: chunk c of sequence s, KV head g; `slot` is its partial slot.
template <int D, int G, bool kWholeStep>
__device__ void decode_item(const DecodeKernelArgs& p, DecodeShared<D, G>& sh, int s, int g, int c, int nchunks,
                            int64_t slot, const ItemInputs<D, G>& in) {
    constexpr int kLanesPerKey = D / 8;
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = lane / kLanesPerKey, dl = lane % kLanesPerKey;
    const int Hq = a.num_q_heads;
    const int k0 = c * p.chunk;
    const int L = clamp_len(in.L_raw, a.max_blocks_per_seq << p.log2_block);
    const int k1 = min(k0 + p.chunk, L);

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }
    wave_steps<D, G, kWholeStep>(p, s, g, k0, k1, in.first_blk, in.qv, lane, wave, m, l, o);

    // ---- wave totals: l over every key lane; o per row, summed by the merge
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] = wave_sum(l[h]);
        *reinterpret_cast<f32x4*>(&sh.o[wave][kq][h][dl * 8]) = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
        *reinterpret_cast<f32x4*>(&sh.o[wave][kq][h][dl * 8 + 4]) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            sh.m[wave][h] = m[h];
            sh.l[wave][h] = l[h];
        }
    }
    __syncthreads();

    // ---- merge the 4 waves: thread -> kElems consecutive outputs of one head
    constexpr int kElems = elems_per_thread<D, G>();
    const int e0 = threadIdx.x * kElems;
    const bool active = e0 < G * D;  // fewer outputs than threads when G * D < 256
    const int h = active ? e0 / D : 0, d0 = active ? e0 % D : 0;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mx = fmaxf(mx, sh.m[w][h]);
    float den = 0.f, val[kElems];
#pragma unroll
    for (int k = 0; k < kElems; ++k) val[k] = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
        const float sc = sh.m[w][h] == -INFINITY ? 0.f : fast_exp2(sh.m[w][h] - mx);  // a wave without keys adds 0
        den += sh.l[w][h] * sc;
#pragma unroll
        for (int k = 0; k < kElems; ++k) {
            float rows = 0.f;
#pragma unroll
            for (int r = 0; r < DecodeShared<D, G>::kRows; ++r) rows += sh.o[w][r][h][d0 + k];
            val[k] += rows * sc;
        }
    }
    const int qh = g * G + h;
    const float inv = 1.f / den;
    if (nchunks == 1) {
        uint16_t* dst = a.out + ((int64_t)s * Hq + qh) * D + d0;
        if (active)
#pragma unroll
            for (int k = 0; k < kElems; ++k) dst[k] = __builtin_bit_cast(uint16_t, (__bf16)(val[k] * inv));
        __syncthreads();  // LDS is reused by the next item
        return;
    }
    if (active && slot < p.max_partials) {
        float* dst = p.part + (slot * Hq + qh) * D + d0;
#pragma unroll
        for (int k = 0; k < kElems; ++k) dst[k] = val[k] * inv;
        if (d0 == 0) p.lse[slot * Hq + qh] = mx + log2f(den);
    }
    __syncthreads();  // LDS is reused by the next item
}

template <int D, int G, bool kWholeStep>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeKernelArgs p, int32_t* prefix_out) {
    __shared__ DecodeShared<D, G> sh;
    const int S = p.a.num_seqs;
    const int Hq = p.a.num_q_heads;
    const int Hkv = p.a.num_kv_heads;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;

    if (!p.persistent) {
        // direct grid: workgroup -> (chunk, sequence, KV head), KV head fastest
        int idx = blockIdx.x;
        const int g = idx % Hkv;
        idx /= Hkv;
        const int s = idx % S;
        const int c = idx / S;
        const ItemInputs<D, G> in = load_item_inputs<D, G>(p, s, g, c);  // before the exit test: one round trip
        const int L = clamp_len(in.L_raw, cap);
        const int n = num_chunks(L, p.chunk);
        if (L == 0 && c == 0)  // a sequence without keys: zero rows
            for (int e = threadIdx.x; e < G * D; e += kDecodeThreads) p.a.out[((int64_t)s * Hq + g * G) * D + e] = 0;
        if (c >= n) return;
        decode_item<D, G, kWholeStep>(p, sh, s, g, c, n, (int64_t)s * p.max_chunks + c, in);
        return;
    }

    extern __shared__ int32_t s_prefix[];  // num_seqs + 1
    chunk_prefix(p, s_prefix, sh.wave_sum);
    if (blockIdx.x == 0) {  // the merge kernel's view of the list; sequences without keys: zero rows
        for (int i = threadIdx.x; i <= S; i += kDecodeThreads) prefix_out[i] = s_prefix[i];
        const int pieces = Hq * D / 8;
        for (int64_t e = threadIdx.x; e < (int64_t)S * pieces; e += kDecodeThreads) {
            const int s = (int)(e / pieces);
            if (s_prefix[s + 1] == s_prefix[s]) store16(p.a.out + e * 8, u32x4{0u, 0u, 0u, 0u});
        }
    }
    // item i = (chunk i / Hkv of the compact list, KV head i % Hkv); the grid is
    // a multiple of 8 workgroups, so a workgroup only meets KV heads congruent
    // to its XCD modulo 8
    const int64_t total_items = (int64_t)s_prefix[S] * Hkv;
    for (int64_t item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int chunk = (int)(item / Hkv);
        const int g = (int)(item - (int64_t)chunk * Hkv);
        int lo = 0, hi = S - 1;  // the sequence owning this chunk: last s with s_prefix[s] <= chunk
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_prefix[mid] <= chunk) lo = mid; else hi = mid - 1;
        }
        const int n = s_prefix[lo + 1] - s_prefix[lo];
        const int c = chunk - s_prefix[lo];
        decode_item<D, G, kWholeStep>(p, sh, lo, g, c, n, chunk, load_item_inputs<D, G>(p, lo, g, c));
    }
}

template <int D, int G, bool kWholeStep>
hipError_t launch_grid(const DecodeKernelArgs& kp, int32_t* prefix, hipStream_t stream) {
    const DecodeArgs& a = kp.a;
    if (!kp.persistent) {
        const int64_t blocks = (int64_t)kp.max_chunks * a.num_seqs * a.num_kv_heads;
        hipLaunchKernelGGL((decode_kernel<D, G, kWholeStep>), dim3((unsigned)blocks), dim3(kDecodeThreads), 0, stream, kp, prefix);
    } else {
        const size_t lds = sizeof(int32_t) * (size_t)(a.num_seqs + 1);
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<D, G, kWholeStep>, kDecodeThreads, lds);
        if (e != hipSuccess) return e;
        if (per_cu < 1) per_cu = 1;
        const int64_t direct = (int64_t)a.num_seqs * kp.max_chunks;
        const int64_t items = (kp.max_partials < direct ? kp.max_partials : direct) * a.num_kv_heads;
        int64_t blocks = (items + kXcds - 1) / kXcds * kXcds;
        int64_t resident = (int64_t)per_cu * device_cu_count() / kXcds * kXcds;
        if (resident < kXcds) resident = kXcds;
        if (blocks > resident) blocks = resident;
        hipLaunchKernelGGL((decode_kernel<D, G, kWholeStep>), dim3((unsigned)blocks), dim3(kDecodeThreads), lds, stream, kp,
                           prefix);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || kp.max_chunks < 2) return e;  // no sequence has two chunks: nothing to merge
    hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3((unsigned)(a.num_seqs * a.num_kv_heads)),
                       dim3(kDecodeThreads), 0, stream, kp, (const int32_t*)prefix);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_typed(const DecodeKernelArgs& kp, int32_t* prefix, hipStream_t stream) {
    // a 64-key step lies in one block when blocks hold >= 64 keys
    if ((1 << kp.log2_block) >= kStepKeys) return launch_grid<D, G, true>(kp, prefix, stream);
    return launch_grid<D, G, false>(kp, prefix, stream);
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
    // chunk: about 4 workgroups per CU-slot's worth of work, 256..8192 keys
    const int64_t key_heads = total * num_kv_heads;
    int chunk = kDecodeWaves * kStepKeys;
    while (chunk < 8192 && (int64_t)chunk * 2 * 4096 <= key_heads) chunk *= 2;
    pl.chunk = chunk;
    pl.max_chunks = (max_seq_len + chunk - 1) / chunk;
    const int64_t direct_items = (int64_t)num_seqs * pl.max_chunks;
    const int64_t real_items = (total + chunk - 1) / chunk + num_seqs;  // bound on chunks actually present
    // a direct grid when its empty workgroups are few (or the launch is small)
    pl.persistent = (direct_items > 2 * real_items && direct_items * num_kv_heads > 4096) ? 1 : 0;
    pl.max_partials = pl.persistent ? (direct_items < real_items ? direct_items : real_items) : direct_items;
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
    kp.max_chunks = pl.max_chunks;
    kp.persistent = pl.persistent;
    kp.max_partials = pl.max_partials;
    char* ws = static_cast<char*>(a.workspace);
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + pl.prefix_offset);
    kp.lse = reinterpret_cast<float*>(ws + pl.lse_offset);
    kp.part = reinterpret_cast<float*>(ws + pl.o_offset);
    kp.qk_scale_log2 = a.scale * kLog2e;
    const int G = a.num_q_heads / a.num_kv_heads;
    if (a.head_dim == 128) {
        switch (G) {
            case 1: return launch_typed<128, 1>(kp, prefix, stream);
            case 2: return launch_typed<128, 2>(kp, prefix, stream);
            case 4: return launch_typed<128, 4>(kp, prefix, stream);
            default: return launch_typed<128, 8>(kp, prefix, stream);
        }
    }
    switch (G) {
        case 1: return launch_typed<64, 1>(kp, prefix, stream);
        case 2: return launch_typed<64, 2>(kp, prefix, stream);
        case 4: return launch_typed<64, 4>(kp, prefix, stream);
        default: return launch_typed<64, 8>(kp, prefix, stream);
    }
}

}  // namespace pkv
