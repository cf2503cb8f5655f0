// paged_gqa_prefill: causal attention of chunks of query rows over a paged KV
// cache, on bf16 MFMA with fp32 accumulation.
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.1 tiles the queries in
// blocks of 128 and, for each, walks only the key blocks at or before it, so the
// full score matrix never exists.  Its per-tile softmax is not exact attention;
// here every query row keeps a running max and sum (online softmax) so the
// result is softmax(QK^T * scale) V exactly up to rounding.
//
// gfx950 design (one workgroup = 4 waves = 128 query rows of one query head):
//  * Each wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A
//    operand, the wave's Q rows stay in registers as the B operand.  In the
//    32x32 result a lane holds one query (column) and 16 keys, so the row max
//    and sum need only the lane and its partner lane 32 away.
//  * The probabilities are already laid out as the B operand of
//    O^T += V^T P^T (keys as the contraction index), so they are packed to bf16
//    in place.  V stays row-major in LDS and the V^T operand is read with
//    ds_read_b64_tr_b16, the gfx950 transposing LDS read.
//  * K/V tiles of 64 keys are copied from the pools straight into LDS with
//    global_load_lds_dwordx4, double-buffered: the loads of tile t+1 are in
//    flight while tile t is computed.  Wave w copies rows [16 w, 16 w + 16) of
//    both tiles; as blocks hold at least 16 keys, those rows sit in one
//    (block, KV head) slab, so the slab address is scalar arithmetic on a
//    block id read with a scalar load one tile ahead, and every lane's offset
//    within the slab is fixed for the whole workgroup.  The LDS tile is
//    unpadded; 16-byte pieces are XOR-swizzled per row so that the K reads
//    (16 rows, one piece) and the transposing V reads (4 rows, four pieces)
//    hit distinct banks.  Every LDS read address is a per-lane register set
//    up once plus a compile-time offset (stage, row block), so the tile loop
//    spends no vector instructions on addressing.  Rows past the last visible
//    key copy a visible row of the same slab (or are zero-filled when the
//    wave's rows hold none), so no unwritten (NaN) slot reaches the MFMA;
//    the causal mask excludes them.
//  * Softmax in the exp2 domain with one FMA per score; the causal mask is
//    applied only on tiles that cross a wave's diagonal; the output is rescaled
//    only when a row maximum grows by more than 2^8 (the weights of a stale
//    maximum stay below 256, exact in fp32 and fine in bf16).  The row sum
//    adds exactly the bf16-rounded weights the MFMA uses (dot with (1, 1)),
//    keeping the output a true weighted average of V rows.
//  * Causal tile skipping: a workgroup stops at its last query's position and
//    a wave skips tiles that lie wholly after its rows (and all compute when
//    it has no rows of the chunk).  Row r of a chunk of n rows on a sequence
//    of length L is at position L - n + r.
//  * Launch order: the longest query tiles first, and the KV head in the low
//    bits of the workgroup index, so that workgroups reading the same K/V land
//    on the same XCD (workgroups are dealt round-robin over the 8 XCDs) and
//    share its L2.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = kPrefillThreads / kWave;
constexpr int kTileQ = 128;  // query rows per workgroup (32 per wave)
constexpr int kTileK = 64;   // keys per LDS tile
constexpr int kWaveRows = kTileK / kPrefillWaves;  // tile rows each wave copies
constexpr float kRescaleSlack = 8.f;             // log2 of the largest stale weight
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // the bf16 pair (1.0, 1.0)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct PrefillKernelArgs {
    PrefillArgs a;
    int32_t log2_block;
    int32_t group;      // query heads per KV head
    int32_t q_tiles;    // tiles of the longest chunk
    float qk_scale_log2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 8 bytes addressed by lanes 4r + i / 4 (r = 0..3).
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
    s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, t);
}

// Slot of 16-byte piece `piece` of LDS tile row `row` (D/8 pieces per row);
// it depends on row % 16 only.  The XOR key maps the 16 rows a K read touches
// (same piece) to 16 different slots, and gives each of the 4 consecutive rows
// a transposing V read touches (4 pieces) its own group of 4 slots, so neither
// read has two lanes on one bank.  An involution: it also names the piece a
// slot holds.
template <int D>
__device__ __forceinline__ int swizzle(int row, int piece) {
    constexpr int kPieces = D / 8;
    return piece ^ ((((row & 3) << 2) | ((row >> 2) & 3)) & (kPieces - 1));
}

// LDS byte address of a __shared__ object (what M0 holds for an LDS DMA).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// global_load_lds_dwordx4 with a scalar base: lane l's 16 bytes at
// base + voff land at LDS byte address lds + 16 l.  Inline asm, so that the
// compiler does not wait for the copies in flight before unrelated LDS reads;
// the loop waits for them explicitly (vmcnt) before its barrier.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// This wave's index, known to the compiler to be the same on every lane.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// What a lane does in the copies and the LDS reads, fixed for the workgroup.
template <int D>
struct Lanes {
    static constexpr int kPieces = D / 8;               // 16-byte pieces per row
    static constexpr int kRowsPerLoad = kWave / kPieces;
    static constexpr int kLoads = kWaveRows / kRowsPerLoad;  // wave loads per matrix and tile
    int row[kLoads];          // copy: row (within the wave's 16) of this lane's 16 bytes
    uint32_t voff[kLoads];    // copy: byte offset of those 16 bytes in the wave's rows of the slab
    int koff[D / 16];         // QK: element offset of this lane's K fragment in a stage, per 16 dims
    int voff_lo[D / 32];      // PV: element offset of this lane's transposing V reads, per 32 dims
    int voff_hi[D / 32];
};

template <int D>
__device__ __forceinline__ Lanes<D> lanes(int lane) {
    using L = Lanes<D>;
    Lanes<D> ln;
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) {
        const int r = i * L::kRowsPerLoad + lane / L::kPieces;
        ln.row[i] = r;
        ln.voff[i] = (uint32_t)(r * D + swizzle<D>(r, lane % L::kPieces) * 8) * 2u;
    }
    const int half = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ln.koff[ks] = r32 * D + swizzle<D>(r32, ks * 2 + half) * 8;
    const int vrow = half * 4 + ((lane & 15) >> 2);
    const int dq = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;  // column within a 32-wide block
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const int d = i * 32 + dq;
        ln.voff_lo[i] = vrow * D + swizzle<D>(vrow, d >> 3) * 8 + (d & 7);
        ln.voff_hi[i] = (vrow + 8) * D + swizzle<D>(vrow + 8, d >> 3) * 8 + (d & 7);
    }
    return ln;
}

// Per-workgroup constants of the tile loop.
template <int D>
struct Loop {
    const PrefillKernelArgs* p;
    const int32_t* table;
    int g, kend, ntiles, wave, lane, qpos, wave_qpos_min, wave_qpos_max;
    bool wave_rows;   // the wave holds at least one row of the chunk
    float c;          // scale * log2 e
    uint16_t* lds;    // [2 stages][K tile, V tile][kTileK][D]
    Lanes<D> ln;
};

template <int D>
constexpr int stage_elems() { return 2 * kTileK * D; }

// Block ids of the slabs holding this wave's rows, a window of 64 tiles at a
// time: lane l holds the id for tile win + l, and a tile's id is read with
// v_readlane.  The window is refilled (one vector load and a wait) only when
// no copy is in flight, so no per-tile memory access waits behind the tile
// copies (vector-memory waits are in issue order).
struct BlockIds {
    int ids;
    int win;
};

template <int D>
__device__ __forceinline__ void fill_ids(const Loop<D>& lp, BlockIds& bi, int t) {
    bi.win = t & ~(kWave - 1);
    const int key = (bi.win + lp.lane) * kTileK + lp.wave * kWaveRows;
    const int idx = min(key >> lp.p->log2_block, lp.p->a.max_blocks_per_seq - 1);
    bi.ids = lp.table[idx];
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), seen by the compiler
}

template <int D>
__device__ __forceinline__ int tile_block(const Loop<D>& lp, BlockIds& bi, int t) {
    if (t - bi.win >= kWave) fill_ids<D>(lp, bi, t);
    return __builtin_amdgcn_readlane(bi.ids, t - bi.win);
}

// Copy this wave's rows of tile kt (K and V) into a stage.  Rows at or past
// kend repeat row kend - 1 of the same slab; a wave with no visible row
// writes zeros instead.
template <int D>
__device__ __forceinline__ void copy_tile(const Loop<D>& lp, int kt, int blk, uint16_t* stage) {
    using L = Lanes<D>;
    const PrefillArgs& a = lp.p->a;
    const int r0 = kt + lp.wave * kWaveRows;  // first key of this wave's rows
    uint16_t* sk = stage + lp.wave * kWaveRows * D;
    uint16_t* sv = sk + kTileK * D;
    const int visible = lp.kend - r0;
    if (visible <= 0) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < L::kLoads; ++i) {
            *reinterpret_cast<u32x4*>(sk + i * L::kRowsPerLoad * D + lp.lane * 8) = zero;
            *reinterpret_cast<u32x4*>(sv + i * L::kRowsPerLoad * D + lp.lane * 8) = zero;
        }
        return;
    }
    const int B = 1 << lp.p->log2_block;
    const int b = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;  // a bad id reads block 0
    const int64_t slab = (((int64_t)b * a.num_kv_heads + lp.g) << lp.p->log2_block) * D + (int64_t)(r0 & (B - 1)) * D;
    const uint16_t* kb = a.k_pool + slab;
    const uint16_t* vb = a.v_pool + slab;
    const uint32_t lk = lds_addr(sk), lv = lds_addr(sv);
    if (visible >= kWaveRows) {
#pragma unroll
        for (int i = 0; i < L::kLoads; ++i) {
            dma16(kb, lp.ln.voff[i], lk + i * kWave * 16);
            dma16(vb, lp.ln.voff[i], lv + i * kWave * 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < L::kLoads; ++i) {
            const int shift = lp.ln.row[i] >= visible ? (lp.ln.row[i] - visible + 1) * D * 2 : 0;
            dma16(kb, lp.ln.voff[i] - shift, lk + i * kWave * 16);
            dma16(vb, lp.ln.voff[i] - shift, lv + i * kWave * 16);
        }
    }
}

// One tile: wait for tile t (stage kCur), start tile t+1 into the other
// stage, then compute tile t.
template <int D, int kCur, bool kNegScale>
__device__ __forceinline__ void tile_step(const Loop<D>& lp, int t, BlockIds& bi, const u32x4 (&qreg)[D / 16],
                                          f32x16 (&acc)[D / 32], float& m, float& lsum) {
    const int kt = t * kTileK;
    const int lane = lp.lane;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of tile t arrived
    __syncthreads();                                    // every wave's have; the other stage is free
    if (t + 1 < lp.ntiles) {
        copy_tile<D>(lp, kt + kTileK, tile_block<D>(lp, bi, t + 1), lp.lds + (kCur ^ 1) * stage_elems<D>());
    }
    if (!lp.wave_rows || kt > lp.wave_qpos_max) return;  // every key of this tile is after this wave's rows
    const float c = lp.c;
    const uint16_t* sk = lp.lds + kCur * stage_elems<D>();
    const uint16_t* sv = sk + kTileK * D;

    // S^T = K Q^T for the two 32-key halves of the tile, interleaved
    f32x16 st[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) st[0][r] = st[1][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(sk + lp.ln.koff[ks]);
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(sk + lp.ln.koff[ks] + 32 * D);
        st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k0), as_bf16x8(qreg[ks]), st[0], 0, 0, 0);
        st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k1), as_bf16x8(qreg[ks]), st[1], 0, 0, 0);
    }
    // read the K fragments three steps (six reads) ahead of their MFMAs, so
    // the LDS latency is hidden behind the MFMAs in flight rather than waited
    // for before each pair
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < D / 8 - 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);

    // scores -> exp2 domain; mask only where the tile crosses this wave's diagonal
    const int half = lane >> 5;
    const bool diag = kt + kTileK - 1 > lp.wave_qpos_min;
    float mt;
    if (diag) {
        mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                const float z = key <= lp.qpos ? st[kb][r] * c : -INFINITY;
                st[kb][r] = z;
                mt = fmaxf(mt, z);
            }
    } else {
        float e = st[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) e = kNegScale ? fminf(e, st[kb][r]) : fmaxf(e, st[kb][r]);
        mt = e * c;
    }
    mt = max_xor32(mt);  // the row's other half is in lane l ^ 32
    // rescale only when a row maximum outgrows the stale one by 2^8
    if (__any(mt > m + kRescaleSlack)) {
        const float m_new = fmaxf(m, mt);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
        m = m_new;
    }
    if (diag) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kb][r] = st[kb][r] == -INFINITY ? 0.f : fast_exp2(st[kb][r] - m);
    } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kb][r] = fast_exp2(__builtin_fmaf(st[kb][r], c, -m));
    }

    // O^T += V^T P^T, 16 keys per MFMA; the row sum adds the same bf16 weights
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            u32x4 pb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pb[i] = pack_bf16x2(st[kb][sub * 8 + 2 * i], st[kb][sub * 8 + 2 * i + 1]);
                ps = dot2_bf16(pb[i], kOnesBf16x2, ps);
            }
            const uint16_t* v16 = sv + (kb * 32 + sub * 16) * D;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const u32x2 lo = lds_read_tr(v16 + lp.ln.voff_lo[i]);
                const u32x2 hi = lds_read_tr(v16 + lp.ln.voff_hi[i]);
                const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb), acc[i], 0, 0, 0);
            }
        }
    lsum += ps;
}

template <int D, bool kNegScale>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillKernelArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * stage_elems<D>()];
    const PrefillArgs& a = p.a;

    // workgroup -> (query tile, sequence, query head); KV head in the low bits
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, S = a.num_seqs;
    int idx = blockIdx.x;
    const int g = idx % Hkv;
    idx /= Hkv;
    const int hg = idx % p.group;
    idx /= p.group;
    const int s = idx % S;
    const int tile = p.q_tiles - 1 - idx / S;
    const int h = g * p.group + hg;

    // rows of this sequence, clamped so that bad offsets never leave q / out
    const int q0 = min(max(a.cu_q_lens[s], 0), a.total_q_tokens);
    const int n = min(min(max(a.cu_q_lens[s + 1], q0), a.total_q_tokens) - q0, a.max_q_len);
    if (tile * kTileQ >= n) return;
    const int cap = a.max_blocks_per_seq << p.log2_block;
    int L = a.seq_lens[s];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int ctx = L - n;  // cached keys before the chunk

    const int lane = threadIdx.x & 63, wave = wave_id(), half = lane >> 5;
    const int qrow = tile * kTileQ + wave * 32 + (lane & 31);  // this lane's query row in the chunk
    const int wave_row0 = tile * kTileQ + wave * 32;

    Loop<D> lp;
    lp.p = &p;
    lp.table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    lp.g = g;
    lp.kend = min(L, ctx + min((tile + 1) * kTileQ, n));  // keys this workgroup may see: [0, kend)
    lp.ntiles = lp.kend > 0 ? (lp.kend + kTileK - 1) / kTileK : 0;
    lp.wave = wave;
    lp.lane = lane;
    lp.qpos = ctx + qrow;  // this lane's absolute position
    lp.wave_qpos_min = ctx + wave_row0;
    lp.wave_qpos_max = ctx + min(wave_row0 + 31, n - 1);
    lp.wave_rows = wave_row0 < n;
    lp.c = p.qk_scale_log2;
    lp.lds = lds;
    lp.ln = lanes<D>(lane);

    u32x4 qreg[D / 16];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint16_t* qp = a.q + ((int64_t)(q0 + qrow) * Hq + h) * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = qrow < n ? load16(qp + ks * 16) : zero;
    }
    // Wait for q here, in a form the compiler's wait placement sees: the
    // tile copies are inline asm it cannot track, so otherwise it would keep
    // a full vector-memory wait before the first MFMA of every tile, which
    // would also wait for the next tile's copies.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    BlockIds bi;
    bi.ids = 0;
    bi.win = 0;
    if (lp.ntiles > 0) {
        fill_ids<D>(lp, bi, 0);
        copy_tile<D>(lp, 0, tile_block<D>(lp, bi, 0), lds);
    }
    for (int t = 0; t < lp.ntiles; t += 2) {
        tile_step<D, 0, kNegScale>(lp, t, bi, qreg, acc, m, lsum);
        if (t + 1 < lp.ntiles) tile_step<D, 1, kNegScale>(lp, t + 1, bi, qreg, acc, m, lsum);
    }

    lsum += __shfl_xor(lsum, 32, kWave);
    if (qrow >= n) return;
    const float inv = (lp.qpos >= 0 && lsum > 0.f) ? 1.f / lsum : 0.f;  // a row with no key is zero
    uint16_t* op = a.out + ((int64_t)(q0 + qrow) * Hq + h) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = i * 32 + j * 8 + half * 4;
            u32x2 w = {pack_bf16x2(acc[i][4 * j] * inv, acc[i][4 * j + 1] * inv),
                       pack_bf16x2(acc[i][4 * j + 2] * inv, acc[i][4 * j + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + d) = w;
        }
}

// ---- small launches: the key range split between two halves of a workgroup
//
// A launch with fewer workgroups than two per CU leaves one wave per SIMD,
// and nothing hides its latencies.  Then a workgroup of 8 waves takes the
// same 128 query rows: waves 0-3 the first half of the key tiles, waves 4-7
// the second, each half streaming its own tiles through its own two stages
// exactly as prefill_kernel does (one workgroup barrier per tile; the half
// with fewer tiles passes its extra barriers idle).  At the end the second
// half hands its running maximum, sum and O^T fragments to the first through
// LDS, and the first merges the two states (each relative to its own
// maximum) and writes the rows.
constexpr int kSplitThreads = 512;

// A tile step for a half that has no tile left: only the barrier.
__device__ __forceinline__ void idle_step() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

template <int D, bool kNegScale>
__global__ __launch_bounds__(kSplitThreads, 2) void prefill_split_kernel(PrefillKernelArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2 * stage_elems<D>()];
    const PrefillArgs& a = p.a;

    // workgroup -> (query tile, sequence, query head), as prefill_kernel
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, S = a.num_seqs;
    int idx = blockIdx.x;
    const int g = idx % Hkv;
    idx /= Hkv;
    const int hg = idx % p.group;
    idx /= p.group;
    const int s = idx % S;
    const int tile = p.q_tiles - 1 - idx / S;
    const int h = g * p.group + hg;

    const int q0 = min(max(a.cu_q_lens[s], 0), a.total_q_tokens);
    const int n = min(min(max(a.cu_q_lens[s + 1], q0), a.total_q_tokens) - q0, a.max_q_len);
    if (tile * kTileQ >= n) return;
    const int cap = a.max_blocks_per_seq << p.log2_block;
    int L = a.seq_lens[s];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int ctx = L - n;

    const int lane = threadIdx.x & 63, wave8 = wave_id(), half = lane >> 5;
    const int part = wave8 >> 2;  // which half of the key tiles
    const int wave = wave8 & 3;   // 32-row block of the tile
    const int qrow = tile * kTileQ + wave * 32 + (lane & 31);
    const int wave_row0 = tile * kTileQ + wave * 32;

    Loop<D> lp;
    lp.p = &p;
    lp.table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    lp.g = g;
    lp.kend = min(L, ctx + min((tile + 1) * kTileQ, n));
    const int T = lp.kend > 0 ? (lp.kend + kTileK - 1) / kTileK : 0;
    const int T0 = T / 2;                    // the first half's tiles: [0, T0); the second's: [T0, T)
    const int tb = part ? T0 : 0, te = part ? T : T0;
    const int steps = T - T0;                // the longer half's tile count: the barriers both halves pass
    lp.ntiles = te;                          // tile_step copies tile t + 1 only while t + 1 < te
    lp.wave = wave;
    lp.lane = lane;
    lp.qpos = ctx + qrow;
    lp.wave_qpos_min = ctx + wave_row0;
    lp.wave_qpos_max = ctx + min(wave_row0 + 31, n - 1);
    lp.wave_rows = wave_row0 < n;
    lp.c = p.qk_scale_log2;
    lp.lds = lds[part];
    lp.ln = lanes<D>(lane);

    u32x4 qreg[D / 16];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint16_t* qp = a.q + ((int64_t)(q0 + qrow) * Hq + h) * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = qrow < n ? load16(qp + ks * 16) : zero;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): q is in (see prefill_kernel)

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    BlockIds bi;
    bi.ids = 0;
    bi.win = 0;
    if (te > tb) {
        fill_ids<D>(lp, bi, tb);
        copy_tile<D>(lp, tb * kTileK, tile_block<D>(lp, bi, tb), lp.lds);
    }
    for (int i = 0; i < steps; i += 2) {
        const int t = tb + i;
        if (t < te)
            tile_step<D, 0, kNegScale>(lp, t, bi, qreg, acc, m, lsum);
        else
            idle_step();
        if (i + 1 < steps) {
            if (t + 1 < te)
                tile_step<D, 1, kNegScale>(lp, t + 1, bi, qreg, acc, m, lsum);
            else
                idle_step();
        }
    }
    lsum += __shfl_xor(lsum, 32, kWave);

    // the second half's state to LDS (the stages are free once every wave is
    // past its last tile), then the first half merges it into its own
    __syncthreads();
    float* xo = reinterpret_cast<float*>(&lds[0][0]);  // [4 waves][D / 32][16][64 lanes]
    float* xm = xo + 4 * (D / 32) * 16 * kWave;        // [4 waves][64 lanes]
    float* xl = xm + 4 * kWave;
    if (part == 1) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) xo[((wave * (D / 32) + i) * 16 + r) * kWave + lane] = acc[i][r];
        xm[wave * kWave + lane] = m;
        xl[wave * kWave + lane] = lsum;
    }
    __syncthreads();
    if (part == 1 || qrow >= n) return;
    const float m1 = xm[wave * kWave + lane], l1 = xl[wave * kWave + lane];
    const float mm = fmaxf(m, m1);
    const float a0 = m == -INFINITY ? 0.f : fast_exp2(m - mm);  // a half without keys adds nothing
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
    lsum = lsum * a0 + l1 * a1;
    const float inv = (lp.qpos >= 0 && lsum > 0.f) ? 1.f / lsum : 0.f;  // a row with no key is zero
    uint16_t* op = a.out + ((int64_t)(q0 + qrow) * Hq + h) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        float o[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = acc[i][r] * a0 + xo[((wave * (D / 32) + i) * 16 + r) * kWave + lane] * a1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = i * 32 + j * 8 + half * 4;
            u32x2 w = {pack_bf16x2(o[4 * j] * inv, o[4 * j + 1] * inv), pack_bf16x2(o[4 * j + 2] * inv, o[4 * j + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + d) = w;
        }
    }
}

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Workgroups a launch needs for two per CU (the plan's CU count, as decode's).
constexpr int64_t kSplitBelow = 2 * 256;

template <int D>
void launch_d(const PrefillKernelArgs& kp, int64_t blocks, hipStream_t stream) {
    if (blocks < kSplitBelow) {
        if (kp.qk_scale_log2 < 0.f)
            hipLaunchKernelGGL((prefill_split_kernel<D, true>), dim3((unsigned)blocks), dim3(kSplitThreads), 0,
                               stream, kp);
        else
            hipLaunchKernelGGL((prefill_split_kernel<D, false>), dim3((unsigned)blocks), dim3(kSplitThreads), 0,
                               stream, kp);
    } else if (kp.qk_scale_log2 < 0.f) {
        hipLaunchKernelGGL((prefill_kernel<D, true>), dim3((unsigned)blocks), dim3(kPrefillThreads), 0, stream, kp);
    } else {
        hipLaunchKernelGGL((prefill_kernel<D, false>), dim3((unsigned)blocks), dim3(kPrefillThreads), 0, stream, kp);
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_q_len == 0 || a.total_q_tokens == 0) return hipSuccess;
    PrefillKernelArgs kp;
    kp.a = a;
    kp.log2_block = ilog2(a.block_size);
    kp.group = a.num_q_heads / a.num_kv_heads;
    kp.q_tiles = (a.max_q_len + kTileQ - 1) / kTileQ;
    kp.qk_scale_log2 = a.scale * kLog2e;
    const int64_t blocks = (int64_t)kp.q_tiles * a.num_seqs * a.num_q_heads;
    if (a.head_dim == 128)
        launch_d<128>(kp, blocks, stream);
    else
        launch_d<64>(kp, blocks, stream);
    return hipGetLastError();
}

}  // namespace pkv
