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
//  * K/V tiles of 64 keys are gathered through the block table straight into
//    LDS with global_load_lds_dwordx4 (no register staging), double-buffered:
//    the loads of tile t+1 are in flight while tile t is computed.  The LDS
//    tile is unpadded; 16-byte pieces are XOR-swizzled per row so that the
//    K reads (16 rows, one piece) and the transposing V reads (4 rows, four
//    pieces) hit distinct banks.  Rows past the last visible key load a copy
//    of a visible row, so no unwritten (NaN) slot reaches the MFMA, and are
//    excluded by the mask.
//  * Softmax in the exp2 domain with one FMA per score; the causal mask is
//    applied only on tiles that cross a wave's diagonal; the output is rescaled
//    only when a row maximum grows by more than 2^8 (the weights of a stale
//    maximum stay below 256, exact in fp32 and fine in bf16).  The row sum
//    adds exactly the bf16-rounded weights the MFMA uses (dot with (1, 1)),
//    keeping the output a true weighted average of V rows.
//  * Causal tile skipping: a workgroup stops at its last query's position and
//    a wave skips tiles that lie wholly after its rows.  Row r of a chunk of n
//    rows on a sequence of length L is at position L - n + r.
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
constexpr float kRescaleSlack = 8.f;             // log2 of the largest stale weight
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // the bf16 pair (1.0, 1.0)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

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

// Slot of 16-byte piece `piece` of LDS tile row `row` (D/8 pieces per row).
// The XOR key maps the 16 rows a K read touches (same piece) to 16 different
// slots, and gives each of the 4 consecutive rows a transposing V read
// touches (4 pieces) its own group of 4 slots, so neither read has two lanes
// on one bank.
template <int D>
__device__ __forceinline__ int swizzle(int row, int piece) {
    constexpr int kPieces = D / 8;
    return piece ^ ((((row & 3) << 2) | ((row >> 2) & 3)) & (kPieces - 1));
}

// Rows of a 64-key tile this wave moves into LDS: rows [16 w, 16 w + 16),
// kLoads wave loads of kRowsPerLoad rows each.
template <int D>
struct TileShare {
    static constexpr int kPieces = D / 8;  // 16-byte pieces per row
    static constexpr int kRowsPerLoad = kWave / kPieces;
    static constexpr int kLoads = kTileK / kPrefillWaves / kRowsPerLoad;
};

// Block ids of this lane's rows of the tile starting at key kt (read one tile
// ahead, so that no table load sits between the LDS-bound loads).  Rows at or
// past kend stand in for row kend - 1, a written row; the mask excludes them.
template <int D>
__device__ __forceinline__ void tile_blocks(const PrefillKernelArgs& p, const int32_t* table, int kt, int kend,
                                            int wave, int lane, int (&blk)[TileShare<D>::kLoads]) {
    using T = TileShare<D>;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        const int row = wave * (kTileK / kPrefillWaves) + i * T::kRowsPerLoad + lane / T::kPieces;
        const int key = min(kt + row, kend - 1);
        blk[i] = table[key >> p.log2_block];
    }
}

// This wave's share of one K/V tile, straight from the pools into LDS.
template <int D>
__device__ __forceinline__ void load_tile(const PrefillKernelArgs& p, int g, int kt, int kend,
                                          const int (&blk)[TileShare<D>::kLoads], uint16_t* sK, uint16_t* sV, int wave,
                                          int lane) {
    using T = TileShare<D>;
    const PrefillArgs& a = p.a;
    const int B = 1 << p.log2_block;
    const int64_t tile = (int64_t)B * D;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        const int row0 = wave * (kTileK / kPrefillWaves) + i * T::kRowsPerLoad;  // first row of this wave load
        const int row = row0 + lane / T::kPieces;
        const int piece = swizzle<D>(row, lane % T::kPieces);  // the piece this lane's LDS slot holds
        const int key = min(kt + row, kend - 1);
        const int b = (unsigned)blk[i] < (unsigned)a.num_blocks ? blk[i] : 0;
        const int64_t off = ((int64_t)b * a.num_kv_heads + g) * tile + (int64_t)(key & (B - 1)) * D + piece * 8;
        __builtin_amdgcn_global_load_lds(a.k_pool + off, (lds_void*)(sK + row0 * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(a.v_pool + off, (lds_void*)(sV + row0 * D), 16, 0, 0);
    }
}

// Per-workgroup constants of the tile loop.
struct RowState {
    int g, kend, ntiles, wave, lane, half, qpos, wave_qpos_min, wave_qpos_max;
    const int32_t* table;
    float c;
};

// One tile of the loop: wait for tile t (stage kCur), start tile t+1 into the
// other stage, then compute tile t.  The stage is a template argument so the
// two stages are distinct LDS objects and the compiler need not wait for the
// loads in flight into one stage before reading the other.
template <int D, int kCur>
__device__ __forceinline__ void tile_step(const PrefillKernelArgs& p, const RowState& rs, int t, uint16_t* sKcur,
                                          uint16_t* sVcur, uint16_t* sKnext, uint16_t* sVnext,
                                          int (&blk)[TileShare<D>::kLoads], const u32x4 (&qreg)[D / 16],
                                          f32x16 (&acc)[D / 32], float& m, float& lsum) {
    const int kt = t * kTileK;
    const int lane = rs.lane, half = rs.half;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(0): this wave's part of tile t (and the next ids) arrived
    __syncthreads();                     // every part is; the other stage is free
    if (t + 1 < rs.ntiles) {
        load_tile<D>(p, rs.g, kt + kTileK, rs.kend, blk, sKnext, sVnext, rs.wave, lane);
        if (t + 2 < rs.ntiles) tile_blocks<D>(p, rs.table, kt + 2 * kTileK, rs.kend, rs.wave, lane, blk);
    }
    if (kt > rs.wave_qpos_max) return;  // every key of this tile is after this wave's rows
    const float c = rs.c;

    // S^T = K Q^T for two 32-key blocks
    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
        const int row = kb * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4 kf = *reinterpret_cast<const u32x4*>(sKcur + row * D + swizzle<D>(row, ks * 2 + half) * 8);
            st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qreg[ks]), st[kb], 0, 0, 0);
        }
    }

    // scores -> exp2 domain; mask only where the tile crosses this wave's diagonal
    const bool diag = kt + kTileK - 1 > rs.wave_qpos_min;
    float mt;
    if (diag) {
        mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                const float z = key <= rs.qpos ? st[kb][r] * c : -INFINITY;
                st[kb][r] = z;
                mt = fmaxf(mt, z);
            }
    } else {
        float hi = st[0][0], lo = st[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                hi = fmaxf(hi, st[kb][r]);
                lo = fminf(lo, st[kb][r]);
            }
        mt = c >= 0.f ? hi * c : lo * c;
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
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
            const int row = kb * 32 + sub * 16 + half * 4 + ((lane & 15) >> 2);
            const int dq = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;  // column within a 32-wide block
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const int d = i * 32 + dq;
                const u32x2 lo = lds_read_tr(sVcur + row * D + swizzle<D>(row, d >> 3) * 8 + (d & 7));
                const u32x2 hi = lds_read_tr(sVcur + (row + 8) * D + swizzle<D>(row + 8, d >> 3) * 8 + (d & 7));
                const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb), acc[i], 0, 0, 0);
            }
        }
    lsum += ps;
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillKernelArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kTileK * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kTileK * D];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kTileK * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kTileK * D];
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

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int qrow = tile * kTileQ + wave * 32 + (lane & 31);  // this lane's query row in the chunk
    const int qpos = ctx + qrow;                                // its absolute position
    const int wave_qpos_min = ctx + tile * kTileQ + wave * 32;
    const int wave_qpos_max = ctx + min(tile * kTileQ + wave * 32 + 31, n - 1);
    const int kend = min(L, ctx + min((tile + 1) * kTileQ, n));  // keys this workgroup may see: [0, kend)
    const int32_t* table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    const float c = p.qk_scale_log2;

    u32x4 qreg[D / 16];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint16_t* qp = a.q + ((int64_t)(q0 + qrow) * Hq + h) * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = qrow < n ? load16(qp + ks * 16) : zero;
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    RowState rs;
    rs.g = g;
    rs.kend = kend;
    rs.ntiles = kend > 0 ? (kend + kTileK - 1) / kTileK : 0;
    rs.wave = wave;
    rs.lane = lane;
    rs.half = half;
    rs.qpos = qpos;
    rs.wave_qpos_min = wave_qpos_min;
    rs.wave_qpos_max = wave_qpos_max;
    rs.table = table;
    rs.c = c;
    int blk[TileShare<D>::kLoads];
    if (rs.ntiles > 0) {
        tile_blocks<D>(p, table, 0, kend, wave, lane, blk);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        load_tile<D>(p, g, 0, kend, blk, sK0, sV0, wave, lane);
        if (rs.ntiles > 1) tile_blocks<D>(p, table, kTileK, kend, wave, lane, blk);
    }
    for (int t = 0; t < rs.ntiles; t += 2) {
        tile_step<D, 0>(p, rs, t, sK0, sV0, sK1, sV1, blk, qreg, acc, m, lsum);
        if (t + 1 < rs.ntiles) tile_step<D, 1>(p, rs, t + 1, sK1, sV1, sK0, sV0, blk, qreg, acc, m, lsum);
    }

    lsum += __shfl_xor(lsum, 32, kWave);
    if (qrow >= n) return;
    const float inv = (qpos >= 0 && lsum > 0.f) ? 1.f / lsum : 0.f;  // a row with no key is zero
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

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
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
        hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)blocks), dim3(kPrefillThreads), 0, stream, kp);
    else
        hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)blocks), dim3(kPrefillThreads), 0, stream, kp);
    return hipGetLastError();
}

}  // namespace pkv
