// Split-K machinery of paged decode shared by the bf16 cache (decode.hip)
// and the INT8 cache (decode_int8.hip): work items, grids, the merge of the
// waves of an item and of the chunks of a sequence.
//
//  * Work item = (sequence, KV head, chunk of `chunk` keys), one workgroup of
//    4 waves.  The chunk is cut into tiles and wave w takes tiles w, w + 4,
//    w + 8, ...; the waves' softmax states are merged through LDS.
//    Short batches use a direct grid over (chunk, sequence, KV head) whose
//    empty items exit at once; long, uneven batches use a persistent grid over
//    a compact item list that each workgroup derives from seq_lens (a block
//    scan in LDS).  Nothing is read back to the host, and the KV head sits in
//    the low bits of the workgroup index, so items of one KV head run on one
//    XCD (workgroups are dealt round-robin over the 8 XCDs) and K/V rows
//    shared between sequences (a common prefix) are re-read from that XCD's L2.
//  * Chunks of a sequence write a normalised partial and its log2-sum-exp,
//    merged in one pass with a running maximum
//    (out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M)).  In a direct grid
//    without packing (small launches) the merge happens inside the split
//    kernel: each chunk stores its partial with agent-scope atomic stores,
//    waits for them to complete, then counts itself in with an agent-scope
//    atomic add, and the chunk that sees the count reach n - 1 loads all
//    partials with agent-scope atomic loads and merges them.  Otherwise (the
//    persistent grid, packed launches) a second kernel merges after a kernel
//    boundary.  A sequence with one chunk is written directly (and the merge
//    kernel is not launched when no sequence can have two); a sequence with
//    no keys gets zeros.
//  * Why the in-kernel hand-off needs no L2 write-back or invalidate: the L2
//    is per XCD and not coherent across XCDs, and the LLVM AMDGPU memory
//    model for this target family (GFX942 and later) makes an agent-scope
//    release "buffer_wbl2 sc1; s_waitcnt vmcnt(0)" and an agent-scope acquire
//    "buffer_inv sc1" -- whole-L2 operations that exist for data moved by
//    non-atomic accesses, which may sit dirty or stale in the L2.  Agent-scope
//    atomic loads, stores and read-modify-writes are themselves coherent at
//    agent scope (the model issues them with sc1, past the XCD's L2), so when
//    every value handed between workgroups is such an access the only part of
//    the release that still matters is the wait for the partial stores to
//    complete before the counter add (vmcnt(0)), and the acquire reduces to
//    issuing the partial loads after the add has returned.  Measured on the
//    8-sequence decode step: with the full fences 18.6 us, without 15.0 us.
#pragma once

#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kDecodeThreads = 256;  // 4 waves share one work item
constexpr int kDecodeWaves = kDecodeThreads / kWave;
constexpr int kStages = 4;           // LDS ring depth of a wave
constexpr int kMaxTilesPerWave = 128;  // ids of a wave's tiles sit in two registers
constexpr int kMaxPersistentSeqs = 2048;  // chunk prefix kept in LDS
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.f;  // log2 of the largest weight a stale running max may give

struct DecodeKernelArgs {
    DecodeArgs a;
    int32_t chunk;       // keys per work item (a multiple of 4 waves' tiles)
    int32_t log2_block;
    int32_t max_chunks;  // chunks of the longest sequence
    int32_t persistent;  // 1: persistent grid over the compact item list
    int32_t pack;        // 1: sequences sharing a chunk are decoded together
    int32_t last_first;  // direct grid: 1 deals the last chunks first
    int32_t* counters;   // direct grid: chunks finished per (sequence, KV head),
                         // the last one merges; null: the merge kernel does
    int64_t max_partials;
    float* lse;         // [max_partials][Hq]
    float* part;        // [max_partials][Hq][D]
    float qk_scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

__device__ __forceinline__ int num_chunks(int L, int chunk) { return L > 0 ? (L + chunk - 1) / chunk : 0; }

// Wait until at most N vector-memory operations of this wave are in flight
// (loads retire in issue order).  The memory clobber keeps the compiler from
// moving LDS reads above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

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

// LDS byte address of a __shared__ object (what M0 holds for an LDS DMA).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// global_load_lds_dwordx4 with a scalar base: lane l's 16 bytes at
// base + voff land at LDS byte address lds + 16 l.  Written as inline asm so
// that the compiler, which cannot tell the four stages apart, does not wait
// for every copy in flight before each LDS read; the ring's waits are
// explicit (wait_vmcnt).  kStream sets the non-temporal hint (nt), used for
// every chunk that is not a shared pack -- rows no other item is known to
// read again -- so that the caches keep what is shared (a packed common
// prefix, q, tables, partials) instead of the stream.  (A launch too small
// to pack may still have sequences on shared blocks; their chunks stream
// with the hint too.)
// Measured with the hint on every chunk that is not a shared pack:
// the 8-sequence decode step 13.6 -> 12.4 us, 16 x 32K private keys
// 381 -> 340 us, the shared-prefix batch 698 -> 626 us; with it on the
// shared packs too that batch took 756 us.
template <bool kStream>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    if (kStream)
        asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
    else
        asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// One wave's running softmax state: O^T fragments (rows = dims, column =
// this lane's head), the head's running max and this lane's share of the sum.
template <int D>
struct WaveState {
    f32x4 acc[D / 16];
    float m;
    float l;
};

// Merge kernel: one workgroup per (sequence, KV head) merges that sequence's
// chunk partials into the bf16 output with a running maximum.  Sequences with
// fewer than two chunks were finished by the split kernel.  The partials are
// loaded kMergeBatch at a time, all of a batch's loads in flight together; in
// the direct grid a sequence's slots start at s * max_chunks whatever its
// length, so the first batch goes out with the length itself and a short
// sequence merges after a single memory round trip.  Slots past the
// sequence's chunk count are loaded (they lie inside the workspace) but never
// used: they may hold anything from earlier launches.
template <int D, int G>
constexpr int elems_per_thread() { return (G * D + kDecodeThreads - 1) / kDecodeThreads; }

constexpr int kMergeBatch = 8;

// One batch of the merge: the lse and output slice of partials
// [base + i0, base + i0 + lim) (lim >= 1), loaded unconditionally (entries past
// lim repeat the batch's last slot) so the batch issues back to back.
// Agent-scope (relaxed) accesses of partials: coherent across the XCDs'
// separate L2 caches (stores write through, loads fetch past the L2), for
// partials merged inside the split kernel by a workgroup on any XCD.
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int kElems, bool kAgent = false>
__device__ __forceinline__ void merge_load(const DecodeKernelArgs& p, int64_t base, int i0, int lim, int qh, int d0,
                                           float (&lb)[kMergeBatch], float (&vb)[kMergeBatch][kElems]) {
    const int Hq = p.a.num_q_heads;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
        const int64_t slot = base + i0 + min(i, lim - 1);
        const float* src = p.part + (slot * Hq + qh) * D + d0;
        if constexpr (kAgent) {
            lb[i] = load_agent(p.lse + slot * Hq + qh);
#pragma unroll
            for (int k = 0; k < kElems; ++k) vb[i][k] = load_agent(src + k);
        } else {
            lb[i] = p.lse[slot * Hq + qh];
#pragma unroll
            for (int k = 0; k < kElems; ++k) vb[i][k] = src[k];
        }
    }
}

// Folds the batch's partials below n into the running (max, sum, numerator).
template <int kElems>
__device__ __forceinline__ void merge_fold(int i0, int n, const float (&lb)[kMergeBatch],
                                           const float (&vb)[kMergeBatch][kElems], float& mx, float& den,
                                           float (&num)[kElems]) {
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
        if (i0 + i < n) {
            const float m_new = fmaxf(mx, lb[i]);
            const float a_old = fast_exp2(mx - m_new);  // 0 on the first partial
            const float w = fast_exp2(lb[i] - m_new);
            den = den * a_old + w;
#pragma unroll
            for (int k = 0; k < kElems; ++k) num[k] = num[k] * a_old + w * vb[i][k];
            mx = m_new;
        }
    }
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_merge_kernel(DecodeKernelArgs p, const int32_t* prefix) {
    constexpr int kElems = elems_per_thread<D, G>();  // outputs per thread
    const int Hkv = p.a.num_kv_heads, Hq = p.a.num_q_heads;
    const int g = blockIdx.x % Hkv, s = blockIdx.x / Hkv;
    const int e0 = threadIdx.x * kElems;
    if (e0 >= G * D) return;
    const int h = e0 / D, d0 = e0 % D;
    const int qh = g * G + h;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;
    // the length (and the persistent grid's first slot) as vector loads
    // issued first: waiting for them leaves a batch issued after them in flight
    int si = s;
    asm volatile("" : "+v"(si));
    const int len = p.a.seq_lens[si];
    const int pre = p.persistent ? prefix[si] : 0;
    // in the direct grid the first batch is bounded by the host's chunk count
    // of the longest sequence (this sequence's slots whatever its length), so
    // it goes out with the length
    float lb[kMergeBatch], vb[kMergeBatch][kElems];
    if (!p.persistent)
        merge_load<D, kElems>(p, (int64_t)s * p.max_chunks, 0, min(p.max_chunks, kMergeBatch), qh, d0, lb, vb);
    const int n = __builtin_amdgcn_readfirstlane(num_chunks(clamp_len(len, cap), p.chunk));
    const int64_t base = p.persistent ? (int64_t)__builtin_amdgcn_readfirstlane(pre) : (int64_t)s * p.max_chunks;
    // slots [base, base + n) must lie in the workspace (else: nothing to merge)
    const bool fits = base + n <= p.max_partials;
    if (p.persistent && fits && n > 0) merge_load<D, kElems>(p, base, 0, min(n, kMergeBatch), qh, d0, lb, vb);
    if (n < 2 || !fits) return;
    float mx = -INFINITY, den = 0.f, num[kElems];
#pragma unroll
    for (int k = 0; k < kElems; ++k) num[k] = 0.f;
    merge_fold<kElems>(0, n, lb, vb, mx, den, num);
    for (int i0 = kMergeBatch; i0 < n; i0 += kMergeBatch) {
        merge_load<D, kElems>(p, base, i0, min(n - i0, kMergeBatch), qh, d0, lb, vb);
        merge_fold<kElems>(i0, n, lb, vb, mx, den, num);
    }
    const float inv = 1.f / den;
    uint16_t* dst = p.a.out + ((int64_t)s * Hq + qh) * D + d0;
#pragma unroll
    for (int k = 0; k < kElems; ++k) dst[k] = __builtin_bit_cast(uint16_t, (__bf16)(num[k] * inv));
}

// This wave's index, known to the compiler to be the same on every lane.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Wait for every vector-memory operation of the wave, in a form the
// compiler's own wait placement sees (so it adds none for those loads later).
__device__ __forceinline__ void wait_all_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0) only

// LDS of one workgroup besides the stages: the waves' softmax states.
template <int D, int G>
struct __attribute__((aligned(16))) DecodeShared {
    float o[kDecodeWaves][G][D];
    float m[kDecodeWaves][G];
    float l[kDecodeWaves][G];
    int32_t wave_sum[kDecodeWaves];
    int32_t ticket;  // the item's place among its sequence's finished chunks
};

// The end of a work item: the waves' states (ws: O^T fragments, lane (j, h)
// holding dims 16 db + 4 j + i of head h) are merged through LDS, and the
// item's result goes out, directly (a sequence with one chunk) or as a
// normalised partial with its log2-sum-exp, merged by the sequence's last
// chunk (direct grid) or by the merge kernel.
template <int D, int G>
__device__ __forceinline__ void finish_item(const DecodeKernelArgs& p, DecodeShared<D, G>& sh, const WaveState<D>& ws,
                                            int s, int g, int nchunks, int64_t slot) {
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int Hq = a.num_q_heads;
    // ---- wave totals: the sum over the head's four lane groups; O^T rows to LDS
    float l = ws.l + __shfl_xor(ws.l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int h = lane & 15, j = lane >> 4;
    if (h < G) {
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(&sh.o[wave][h][16 * db + 4 * j]) = ws.acc[db];
        if (j == 0) {
            sh.m[wave][h] = ws.m;
            sh.l[wave][h] = l;
        }
    }
    __syncthreads();

    // ---- merge the 4 waves: thread -> kElems consecutive outputs of one head
    constexpr int kElems = elems_per_thread<D, G>();
    const int e0 = threadIdx.x * kElems;
    const bool active = e0 < G * D;  // fewer outputs than threads when G * D < 256
    const int hh = active ? e0 / D : 0, d0 = active ? e0 % D : 0;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) mx = fmaxf(mx, sh.m[v][hh]);
    float den = 0.f, val[kElems];
#pragma unroll
    for (int k = 0; k < kElems; ++k) val[k] = 0.f;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) {
        const float sc = sh.m[v][hh] == -INFINITY ? 0.f : fast_exp2(sh.m[v][hh] - mx);  // a wave without keys adds 0
        den += sh.l[v][hh] * sc;
#pragma unroll
        for (int k = 0; k < kElems; ++k) val[k] += sh.o[v][hh][d0 + k] * sc;
    }
    const int qh = g * G + hh;
    const float inv = 1.f / den;
    if (nchunks == 1) {
        uint16_t* dst = a.out + ((int64_t)s * Hq + qh) * D + d0;
        if (active)
#pragma unroll
            for (int k = 0; k < kElems; ++k) dst[k] = __builtin_bit_cast(uint16_t, (__bf16)(val[k] * inv));
        __syncthreads();  // LDS is reused by the next item
        return;
    }
    if (!p.counters) {  // partials for the merge kernel
        if (active && slot < p.max_partials) {
            float* dst = p.part + (slot * Hq + qh) * D + d0;
#pragma unroll
            for (int k = 0; k < kElems; ++k) dst[k] = val[k] * inv;
            if (d0 == 0) p.lse[slot * Hq + qh] = mx + log2f(den);
        }
        __syncthreads();  // LDS is reused by the next item
        return;
    }
    // direct grid, no merge kernel: the partial goes out with agent-scope
    // stores, which complete (vmcnt) only once visible at the device's point
    // of coherence; after every thread's have, the chunk is counted in with an
    // agent-scope atomic, and the sequence's last chunk to arrive reads all
    // partials (slots s * max_chunks + c, c < n) with agent-scope loads issued
    // after the count returned, merges them and puts the counter back to zero.
    // Every value handed between workgroups is an agent-scope access, so no
    // L2 write-back or invalidate (the release / acquire fences) is needed.
    const int n = min(nchunks, p.max_chunks);  // chunks the grid holds
    if (active) {
        float* dst = p.part + (slot * Hq + qh) * D + d0;
#pragma unroll
        for (int k = 0; k < kElems; ++k) store_agent(dst + k, val[k] * inv);
        if (d0 == 0) store_agent(p.lse + slot * Hq + qh, mx + log2f(den));
    }
    wait_all_vm();
    __syncthreads();
    int32_t* cnt = p.counters + (int64_t)s * a.num_kv_heads + g;
    if (threadIdx.x == 0) sh.ticket = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sh.ticket == n - 1) {
        if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (active) {
            const int64_t base = (int64_t)s * p.max_chunks;
            float lb[kMergeBatch], vb[kMergeBatch][kElems];
            float m2 = -INFINITY, den2 = 0.f, num[kElems];
#pragma unroll
            for (int k = 0; k < kElems; ++k) num[k] = 0.f;
            for (int i0 = 0; i0 < n; i0 += kMergeBatch) {
                merge_load<D, kElems, true>(p, base, i0, min(n - i0, kMergeBatch), qh, d0, lb, vb);
                merge_fold<kElems>(i0, n, lb, vb, m2, den2, num);
            }
            const float inv2 = 1.f / den2;
            uint16_t* dst = a.out + ((int64_t)s * Hq + qh) * D + d0;
#pragma unroll
            for (int k = 0; k < kElems; ++k) dst[k] = __builtin_bit_cast(uint16_t, (__bf16)(num[k] * inv2));
        }
    }
    __syncthreads();  // LDS is reused by the next item
}

// ---- sequences sharing a chunk (a common prefix: aliased blocks)
//
// The MFMA tiles have 16 columns and a group fills G of them, so up to
// P = 16 / G sequences whose chunk c is the same physical K/V (every block of
// the chunk equal) are decoded by one item, in columns [j G, (j + 1) G) for
// the pack's j-th sequence: the chunk is read once instead of P times.  The
// pack of chunk c is fixed per aligned run of P sequences starting at
// lead = s - s % P: sequence lead + j joins when lead and it both hold keys
// past the chunk (so neither's new row of a decode_append is in it, and both
// write partials) and its chunk's block ids equal lead's.  Every item of the
// run evaluates the same predicate on the same data, so the members' own
// items know to exit, with no communication.  Only chunks of whole blocks
// whose P x (blocks per chunk) ids fit one load per lane are considered, and only in launches
// with more items than two rounds of resident workgroups: below that every
// item runs at once, a pack does not shorten the step, and its loads and
// ballots lengthen each item's start.

template <int G>
constexpr int pack_width() { return 16 / G; }

// What an item loads for the predicate: lane j < P the length of sequence
// lead + j, lane l < P nb the id of block l % nb of sequence lead + l / nb.
struct PackInputs {
    int len;
    int id;
    bool on;  // this chunk is considered for packing
};

template <int G>
__device__ __forceinline__ PackInputs load_pack_inputs(const DecodeKernelArgs& p, int s, int c) {
    constexpr int P = pack_width<G>();
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63;
    const int nb = p.chunk >> p.log2_block;
    PackInputs pk;
    pk.on = p.pack && P > 1 && (p.chunk & ((1 << p.log2_block) - 1)) == 0 && P * nb <= kWave;
    pk.len = 0;
    pk.id = -1;
    if (!pk.on) return pk;
    const int lead = s - s % P;
    if (lane < P && lead + lane < a.num_seqs) pk.len = a.seq_lens[lead + lane];
    const int js = lane / nb, b = (c * p.chunk >> p.log2_block) + lane % nb;
    if (lane < P * nb && lead + js < a.num_seqs && b < a.max_blocks_per_seq)
        pk.id = a.block_table[(int64_t)(lead + js) * a.max_blocks_per_seq + b];
    return pk;
}

// The pack of chunk c for the run of s (bit j: sequence lead + j; 0 when no
// sequence joins lead).  Needs pk's loads to have landed.
template <int G>
__device__ __forceinline__ uint32_t pack_of(const DecodeKernelArgs& p, const PackInputs& pk, int c) {
    constexpr int P = pack_width<G>();
    if (!pk.on) return 0;
    const int lane = threadIdx.x & 63;
    const int nb = p.chunk >> p.log2_block;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;
    const int after = (c + 1) * p.chunk;  // both need keys past the chunk
    const uint64_t long_enough = __ballot(lane < P && clamp_len(pk.len, cap) > after);
    const int lead_id = __shfl(pk.id, lane % nb, kWave);
    const uint64_t same = __ballot(lane < P * nb && pk.id == lead_id && pk.id >= 0);
    if (!(long_enough & 1)) return 0;
    const uint64_t all = nb == 64 ? ~0ull : ((1ull << nb) - 1);
    uint32_t pack = 0;
    for (int j = 1; j < P; ++j)
        if (((long_enough >> j) & 1) && ((same >> (j * nb)) & all) == all) pack |= 1u << j;
    return pack ? pack | 1u : 0u;
}

// The end of a packed item: as finish_item, for the 16 columns of the pack's
// sequences, through LDS that the stages no longer need (o: [waves][16][D]
// floats in obuf, the waves' maxima and sums in ml); each member writes the
// normalised partial and log2-sum-exp of chunk c to its own slot.
template <int D, int G>
__device__ __forceinline__ void finish_pack(const DecodeKernelArgs& p, float* obuf, float* ml, const WaveState<D>& ws,
                                            int lead, int g, int c, uint32_t pack) {
    extern __shared__ int32_t s_prefix[];  // the persistent grid's chunk prefix
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int Hq = a.num_q_heads;
    float l = ws.l + __shfl_xor(ws.l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    __syncthreads();  // every wave is past its tiles: the stages are free
    const int h = lane & 15, j = lane >> 4;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4*>(&obuf[(wave * 16 + h) * D + 16 * db + 4 * j]) = ws.acc[db];
    if (j == 0) {
        ml[wave * 16 + h] = ws.m;
        ml[kDecodeWaves * 16 + wave * 16 + h] = l;
    }
    __syncthreads();
    constexpr int kElems = 16 * D / kDecodeThreads;
    const int e0 = threadIdx.x * kElems, col = e0 / D, d0 = e0 % D;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) mx = fmaxf(mx, ml[v * 16 + col]);
    float den = 0.f, val[kElems];
#pragma unroll
    for (int k = 0; k < kElems; ++k) val[k] = 0.f;
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) {
        const float mv = ml[v * 16 + col];
        const float sc = mv == -INFINITY ? 0.f : fast_exp2(mv - mx);
        den += ml[kDecodeWaves * 16 + v * 16 + col] * sc;
#pragma unroll
        for (int k = 0; k < kElems; ++k) val[k] += obuf[(v * 16 + col) * D + d0 + k] * sc;
    }
    const int js = col / G;
    if ((pack >> js) & 1) {
        const int seq = lead + js;
        const int64_t slot = p.persistent ? (int64_t)s_prefix[seq] + c : (int64_t)seq * p.max_chunks + c;
        const int qh = g * G + col % G;
        if (slot < p.max_partials) {
            const float inv = 1.f / den;
            float* dst = p.part + (slot * Hq + qh) * D + d0;
#pragma unroll
            for (int k = 0; k < kElems; ++k) dst[k] = val[k] * inv;
            if (d0 == 0) p.lse[slot * Hq + qh] = mx + log2f(den);
        }
    }
    __syncthreads();  // LDS is reused by the next item
}

// The grid of a decode kernel: the direct grid (workgroup -> one item) or
// the persistent one (workgroups walk the compact item list).  load(s, g, c)
// fetches what an item needs before its first K/V load; run(s, g, c, n,
// slot, inputs, prefetch) computes the item and calls prefetch() once its own inputs
// are in, which lets the next item's inputs travel with its first tiles.
template <int D, int G, typename Load, typename Run>
__device__ __forceinline__ void run_items(const DecodeKernelArgs& p, DecodeShared<D, G>& sh, int32_t* prefix_out,
                                          Load load, Run run) {
    const int S = p.a.num_seqs;
    const int Hq = p.a.num_q_heads;
    const int Hkv = p.a.num_kv_heads;
    const int cap = p.a.max_blocks_per_seq << p.log2_block;

    if (!p.persistent) {
        // direct grid: workgroup -> (chunk, sequence, KV head), KV head
        // fastest; in a one-round launch the last chunks first: they are
        // mostly empty and leave at once, so when the grid is larger than
        // the resident workgroups the real items are not dispatched behind
        // them
        int idx = blockIdx.x;
        const int g = idx % Hkv;
        idx /= Hkv;
        const int s = idx % S;
        const int c = p.last_first ? p.max_chunks - 1 - idx / S : idx / S;
        const auto in = load(s, g, c);  // before the exit test: one round trip
        const int L = clamp_len(in.L_raw, cap);
        const int n = num_chunks(L, p.chunk);
        if (L == 0 && c == 0)  // a sequence without keys: zero rows
            for (int e = threadIdx.x; e < G * D; e += kDecodeThreads) p.a.out[((int64_t)s * Hq + g * G) * D + e] = 0;
        if (c >= n) return;
        run(s, g, c, n, (int64_t)s * p.max_chunks + c, in, [] {});
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
    struct Item {
        int s, g, c, n, chunk;
    };
    auto locate = [&](int64_t item) {
        Item it;
        it.chunk = (int)(item / Hkv);
        it.g = (int)(item - (int64_t)it.chunk * Hkv);
        int lo = 0, hi = S - 1;  // the sequence owning this chunk: last s with s_prefix[s] <= chunk
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_prefix[mid] <= it.chunk) lo = mid; else hi = mid - 1;
        }
        it.s = lo;
        it.n = s_prefix[lo + 1] - s_prefix[lo];
        it.c = it.chunk - s_prefix[lo];
        return it;
    };
    int64_t item = blockIdx.x;
    if (item >= total_items) return;
    Item cur = locate(item);
    auto in = load(cur.s, cur.g, cur.c);
    for (; item < total_items; item += gridDim.x) {
        const int64_t nxt = item + gridDim.x;
        Item next = cur;
        auto in_next = in;
        run(cur.s, cur.g, cur.c, cur.n, (int64_t)cur.chunk, in, [&] {
            if (nxt < total_items) {
                next = locate(nxt);
                in_next = load(next.s, next.g, next.c);
            }
        });
        cur = next;
        in = in_next;
    }
}

// Launch a split kernel over its grid, then the merge kernel if a sequence
// can have two chunks.
typedef void (*SplitKernel)(DecodeKernelArgs, int32_t*);

template <int D, int G>
hipError_t launch_split(SplitKernel kernel, const DecodeKernelArgs& kp, int32_t* prefix, hipStream_t stream) {
    const DecodeArgs& a = kp.a;
    if (!kp.persistent) {
        const int64_t blocks = (int64_t)kp.max_chunks * a.num_seqs * a.num_kv_heads;
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kDecodeThreads), 0, stream, kp, prefix);
    } else {
        const size_t lds = sizeof(int32_t) * (size_t)(a.num_seqs + 1);
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeThreads, lds);
        if (e != hipSuccess) return e;
        if (per_cu < 1) per_cu = 1;
        const int64_t direct = (int64_t)a.num_seqs * kp.max_chunks;
        const int64_t items = (kp.max_partials < direct ? kp.max_partials : direct) * a.num_kv_heads;
        int64_t blocks = (items + kXcds - 1) / kXcds * kXcds;
        int64_t resident = (int64_t)per_cu * device_cu_count() / kXcds * kXcds;
        if (resident < kXcds) resident = kXcds;
        if (blocks > resident) blocks = resident;
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kDecodeThreads), lds, stream, kp, prefix);
    }
    hipError_t e = hipGetLastError();
    // no sequence has two chunks, or the split kernel merges: no merge kernel
    if (e != hipSuccess || kp.max_chunks < 2 || kp.counters) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3((unsigned)(a.num_seqs * a.num_kv_heads)),
                       dim3(kDecodeThreads), 0, stream, kp, (const int32_t*)prefix);
    return hipGetLastError();
}

inline int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

}  // namespace
}  // namespace pkv
