// paged_gqa_decode_int8: decode over an INT8 KV cache.
//
// "从零搭建AI工程能力：手写KV Cache与动态批处理实战" section 3.2 stores the KV
// cache as 8-bit integers instead of 16-bit floats, half the bytes; decode is
// bound by HBM bandwidth and reads every cached byte once per step, so half
// the bytes is up to twice the step rate.  The cache holds codes
// [num_blocks][num_kv_heads][block_size][head_dim] int8 and one fp32 scale per
// (block, KV head, slot) for K and for V; a row stands for code * scale.
//
// Items, grids and merges are those of decode_common.h; the tile differs from
// the bf16 kernel's:
//  * A tile is 32 keys of one block (block_size >= 32): 32 rows of K codes,
//    32 of V codes and their 2 x 32 scales, 8.25 KB at D = 128 (the bytes of
//    a 16-key bf16 tile), copied by global_load_lds_dwordx4 into the wave's
//    LDS ring as in the bf16 kernel.
//  * Codes become bf16 MFMA operands exactly (|code| <= 127): a signed byte
//    to fp32 conversion per code and one pack per two.  The scales stay off
//    the matrix cores: S^T = (K_codes Q^T) times each key's k_scale, and each
//    key's v_scale multiplies its softmax weight (P' = P v_scale), so that
//    O^T = V_codes^T P'^T.  P' goes to the matrix cores as two bf16 parts,
//    hi = bf16(P') and lo = bf16(P' - hi), one MFMA each, so the weights keep
//    16 significant bits and the running sum, which adds the unscaled
//    weights, divides the same weights out: the output is a convex
//    combination of the dequantised rows.
//  * S^T of each 16-key half: v_mfma_f32_16x16x32_bf16, lane (key i, group j)
//    holding dims [j D/4, (j + 1) D/4) of its key row (the Q fragments follow
//    the same dim order).  The 8 weights a lane then holds (keys 4j..4j+3 of
//    both halves, for its head) are the B operand of one 16x16x32 MFMA per 16
//    dims of O^T; its A operand, 8 keys of one dim per lane, comes straight
//    from LDS with ds_read_b64_tr_b8.
//  * Keys past the sequence end are masked to -inf and their v_scale taken
//    as 0, so neither an unwritten code (any byte is a finite code) nor an
//    unwritten scale (possibly NaN) reaches the result.
//  * Sequences whose chunk is the same physical blocks (a shared prefix)
//    are decoded together in the MFMA's spare columns, as in the bf16 kernel
//    (decode_common.h): the chunk's codes are read and converted once for
//    the whole pack instead of once per sequence.
//  * decode_append_int8 folds the step's kv_append_int8 into the launch, as
//    decode_append does for bf16: every workgroup quantises its sequence's
//    new row (its lanes hold the row, the row maximum is a butterfly), and
//    the wave whose tile holds key L - 1 writes codes and scales to the cache
//    and patches them into its LDS stage once the tile's copy has landed.
#include "decode_common.h"

namespace pkv {
namespace {

constexpr int kTile8 = kDecodeInt8TileKeys;  // keys per tile and per LDS stage of a wave
constexpr int kInt8PackedChunk = 2048;       // keys per work item when sequences are packed

typedef int i32x2_t __attribute__((vector_size(2 * sizeof(int))));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

// LDS slot of 16-byte piece `piece` of stage row `row` (an involution).  Rows
// are D bytes, 256 / D of them per bank sweep; the K reads (16 rows, one
// piece) and the transposing V reads (rows 4j..4j+3 and 16+4j..16+4j+3, one
// piece) then put every 16-byte access of a 16-lane group on its own banks.
template <int D>
__device__ __forceinline__ int swz8(int row, int piece) {
    constexpr int kPieces = D / 16, kShift = D == 128 ? 1 : 2;
    return piece ^ (((row >> kShift) & (kPieces - 1)) ^ (((row >> 4) & 1) * (kPieces / 2)));
}

// What a lane does with a tile, fixed for the whole item.
template <int D>
struct Int8Lanes {
    static constexpr int kPieces = D / 16;                  // 16-byte pieces per code row
    static constexpr int kRowsPerLoad = kWave / kPieces;
    static constexpr int kLoads = kTile8 / kRowsPerLoad;     // wave loads per code matrix and tile
    static constexpr int kDma = 2 * kLoads + 1;              // K, V and one for both scale rows
    static constexpr int kChunk = kPieces / 4;               // 16-byte reads of K codes per half tile
    uint32_t dma_off[kLoads];  // DMA: byte offset of this lane's piece within the tile's rows
    int k_off[2][kChunk];      // QK: LDS byte offset of this lane's K codes, per half and read
    int v_off[D / 16];         // PV: LDS byte offset of this lane's transposing read, per 16 dims
};

template <int D>
__device__ __forceinline__ Int8Lanes<D> int8_lanes(int lane) {
    using T = Int8Lanes<D>;
    Int8Lanes<D> tl;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        const int row = i * T::kRowsPerLoad + lane / T::kPieces;
        tl.dma_off[i] = (uint32_t)(row * D + swz8<D>(row, lane % T::kPieces) * 16);
    }
    const int j = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int u = 0; u < T::kChunk; ++u) {
            const int row = 16 * hf + i16;
            tl.k_off[hf][u] = row * D + swz8<D>(row, j * T::kChunk + u) * 16;
        }
    // lanes 2r and 2r + 1 of a group address the two halves of one piece of
    // key row 4j + r (r < 4) or 16 + 4j + r - 4; lane i then receives dim i of
    // those 8 keys
    const int r = i16 >> 1, b = i16 & 1;
    const int key = r < 4 ? 4 * j + r : 16 + 4 * j + (r - 4);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) tl.v_off[db] = key * D + swz8<D>(key, db) * 16 + 8 * b;
    return tl;
}

// The LDS stages of the block's waves (a ring of R): codes and the scale rows.
template <int D>
struct Int8Stages {
    int8_t* k[kStages];
    int8_t* v[kStages];
    float* sc[kStages];  // per wave: 32 K scales, then 32 V scales
};

// global_load_lds_dwordx4 with a per-lane 64-bit address (the scale rows of K
// and V live in different arrays): lane l's 16 bytes land at lds + 16 l.
// kStream: the non-temporal hint, as dma16.
template <bool kStream>
__device__ __forceinline__ void dma16_addr(const void* addr, uint32_t lds) {
    if (kStream)
        asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(addr), "{m0}"(lds) : "memory");
    else
        asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(addr), "{m0}"(lds) : "memory");
}

// Per-wave view of the item.
template <int D>
struct Int8WaveItem {
    const DecodeArgs* a;
    int log2_block, g, k0, kend, wave, lane, n_tiles;
    int ids0, ids1;  // block id of tile t in lane t % 64 of ids(t / 64)
    int L;           // keys of the sequence
    bool stream;     // not a shared pack: load the chunk's rows with the non-temporal hint
    bool append;     // decode_append_int8: the new row (this lane's codes, the scales) is key L - 1
    u32x2 kq, vq;
    float ks_new, vs_new;
    float c;         // scale * log2 e
    u32x4 qf[D / 32];
    Int8Lanes<D> tl;
    Int8Stages<D> st;
};

template <int D>
__device__ __forceinline__ int tile_blk8(const Int8WaveItem<D>& w, int t) {
    const int v = t < kWave ? w.ids0 : w.ids1;
    return __builtin_amdgcn_readlane(v, t & (kWave - 1));
}

template <int D>
__device__ __forceinline__ int tile_key8(const Int8WaveItem<D>& w, int t) {
    return w.k0 + kTile8 * (w.wave + kDecodeWaves * t);
}

// Copy tile t (keys [kt, kt + 32) of one block) into a stage: the code rows
// of K and V and, from lanes 0..15, the two 128-byte scale rows.  Rows past
// the sequence end are copied too (they stay inside the block) and masked by
// the consumer.  kStream: load with the non-temporal hint.
template <int D, bool kStream>
__device__ __forceinline__ void issue8_tile(const Int8WaveItem<D>& w, int t, int stage) {
    using T = Int8Lanes<D>;
    const DecodeArgs& a = *w.a;
    const int blk = tile_blk8(w, t);
    const int b = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;  // a bad id reads block 0, masked below
    const int B = 1 << w.log2_block;
    const int64_t row0 = ((int64_t)b * a.num_kv_heads + w.g) * B + (tile_key8(w, t) & (B - 1));
    const int8_t* kb = a.k_codes + row0 * D;
    const int8_t* vb = a.v_codes + row0 * D;
    const uint32_t wave_bytes = (uint32_t)(w.wave * kTile8 * D);
    const uint32_t sk = lds_addr(w.st.k[stage]) + wave_bytes, sv = lds_addr(w.st.v[stage]) + wave_bytes;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        dma16<kStream>(kb, w.tl.dma_off[i], sk + i * kWave * 16);
        dma16<kStream>(vb, w.tl.dma_off[i], sv + i * kWave * 16);
    }
    if (w.lane < 16) {
        const float* src = (w.lane < 8 ? a.k_scales : a.v_scales) + row0 + 4 * (w.lane & 7);
        dma16_addr<kStream>(src, lds_addr(w.st.sc[stage]) + (uint32_t)(w.wave * 2 * kTile8 * 4));
    }
}

template <int D>
__device__ __forceinline__ void issue8(const Int8WaveItem<D>& w, int t, int stage) {
    if (w.stream)
        issue8_tile<D, true>(w, t, stage);
    else
        issue8_tile<D, false>(w, t, stage);
}

// decode_append_int8, on the tile holding key L - 1 (row r0 of the tile):
// the new row's codes and scales replace that row of the wave's stage (its
// copy may predate the store) and go to the cache.
template <int D>
__device__ __forceinline__ void put_new_row8(const Int8WaveItem<D>& w, int t, int kS) {
    constexpr int kHalves = D / 8;  // 8-byte halves of 16-byte pieces per code row; one per lane
    const int r0 = w.L - 1 - tile_key8(w, t);
    const int p = w.lane % kHalves;
    const int off = r0 * D + swz8<D>(r0, p / 2) * 16 + (p & 1) * 8;
    if (w.lane < kHalves) {
        *reinterpret_cast<u32x2*>(w.st.k[kS] + w.wave * kTile8 * D + off) = w.kq;
        *reinterpret_cast<u32x2*>(w.st.v[kS] + w.wave * kTile8 * D + off) = w.vq;
    }
    float* ss = w.st.sc[kS] + w.wave * 2 * kTile8;
    if (w.lane == 0) {
        ss[r0] = w.ks_new;
        ss[kTile8 + r0] = w.vs_new;
    }
    const int blk = tile_blk8(w, t);
    if ((unsigned)blk < (unsigned)w.a->num_blocks && w.lane < 2 * kHalves) {
        const int B = 1 << w.log2_block;
        const int64_t row = ((int64_t)blk * w.a->num_kv_heads + w.g) * B + ((w.L - 1) & (B - 1));
        if (w.lane < kHalves) {
            *reinterpret_cast<u32x2*>(w.a->k_codes_w + row * D + p * 8) = w.kq;
            if (p == 0) w.a->k_scales_w[row] = w.ks_new;
        } else {
            *reinterpret_cast<u32x2*>(w.a->v_codes_w + row * D + p * 8) = w.vq;
            if (p == 0) w.a->v_scales_w[row] = w.vs_new;
        }
    }
}

// Eight int8 codes (two dwords, in order) -> eight bf16 (exact).
__device__ __forceinline__ u32x4 codes_to_bf16(uint32_t lo, uint32_t hi) {
    auto cv = [](uint32_t w, int k) { return (float)((int32_t)(w << (24 - 8 * k)) >> 24); };
    return u32x4{pack_bf16x2(cv(lo, 0), cv(lo, 1)), pack_bf16x2(cv(lo, 2), cv(lo, 3)),
                 pack_bf16x2(cv(hi, 0), cv(hi, 1)), pack_bf16x2(cv(hi, 2), cv(hi, 3))};
}

__device__ __forceinline__ bf16x8 as_bf16x8_8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Tile t from stage kS of a ring of R (all R stages in flight): wait for it,
// S^T, softmax, O^T, then refill its stage with tile t + R.
template <int D, int R, int kS>
__device__ __forceinline__ void tile_step8(const Int8WaveItem<D>& w, int t, WaveState<D>& ws) {
    using T = Int8Lanes<D>;
    constexpr int kDma = T::kDma;
    static_assert(R == 2 || R == 4, "ring depth");
    const int after = min(R - 1, w.n_tiles - 1 - t);  // tiles issued after t
    if (after >= 3) wait_vmcnt<3 * kDma>();
    else if (after == 2) wait_vmcnt<2 * kDma>();
    else if (after == 1) wait_vmcnt<kDma>();
    else wait_vmcnt<0>();
    if (w.append && w.kend == w.L && tile_key8(w, t) + kTile8 >= w.kend) put_new_row8<D>(w, t, kS);

    // every LDS read of the tile goes out before the first MFMA waits on one
    const int8_t* sk = w.st.k[kS] + w.wave * kTile8 * D;
    const int8_t* sv = w.st.v[kS] + w.wave * kTile8 * D;
    const float* ss = w.st.sc[kS] + w.wave * 2 * kTile8;
    const int j = w.lane >> 4;
    u32x4 kc[2][T::kChunk];
    u32x2 vc[D / 16];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int u = 0; u < T::kChunk; ++u) kc[hf][u] = *reinterpret_cast<const u32x4*>(sk + w.tl.k_off[hf][u]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        vc[db] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                               (lds_i32x2*)(sv + w.tl.v_off[db])));
    const f32x4 ks0 = *reinterpret_cast<const f32x4*>(ss + 4 * j);
    const f32x4 ks1 = *reinterpret_cast<const f32x4*>(ss + 16 + 4 * j);
    const f32x4 vs0 = *reinterpret_cast<const f32x4*>(ss + kTile8 + 4 * j);
    const f32x4 vs1 = *reinterpret_cast<const f32x4*>(ss + kTile8 + 16 + 4 * j);
    __builtin_amdgcn_sched_barrier(0);

    // S^T of both halves; MFMA c reads bytes [8c, 8c + 8) of the lane's codes
    f32x4 s[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        s[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            const u32x4 q4 = kc[hf][c / 2];
            const u32x4 a = (c & 1) ? codes_to_bf16(q4[2], q4[3]) : codes_to_bf16(q4[0], q4[1]);
            s[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_8(a), as_bf16x8_8(w.qf[c]), s[hf], 0, 0, 0);
        }
    }

    // lane (j, h) holds the scores of keys kt + 16 hf + 4j + r for head h
    const int kt = tile_key8(w, t);
    const bool ok_blk = (unsigned)tile_blk8(w, t) < (unsigned)w.a->num_blocks;
    float z[8], vs[8];
    if (ok_blk && kt + kTile8 <= w.kend) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            z[r] = s[0][r] * (ks0[r] * w.c);
            z[4 + r] = s[1][r] * (ks1[r] * w.c);
            vs[r] = vs0[r];
            vs[4 + r] = vs1[r];
        }
    } else {
        const int key0 = kt + 4 * j;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok0 = ok_blk && key0 + r < w.kend, ok1 = ok_blk && key0 + 16 + r < w.kend;
            z[r] = ok0 ? s[0][r] * (ks0[r] * w.c) : -INFINITY;
            z[4 + r] = ok1 ? s[1][r] * (ks1[r] * w.c) : -INFINITY;
            vs[r] = ok0 ? vs0[r] : 0.f;
            vs[4 + r] = ok1 ? vs1[r] : 0.f;
        }
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    if (__any(mx > ws.m + kRescaleSlack)) {
        float mh = fmaxf(mx, __shfl_xor(mx, 16, kWave));  // the head's max over the tile
        mh = fmaxf(mh, __shfl_xor(mh, 32, kWave));
        const float m_new = fmaxf(ws.m, mh);
        const float alpha = fast_exp2(ws.m - m_new);  // 0 while m is -inf
        ws.l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) ws.acc[db] *= alpha;
        ws.m = m_new;
    }
    // a head whose tile is all masked keeps m = -inf and gets zero weights
    const float mref = ws.m == -INFINITY ? 0.f : ws.m;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(z[i] - mref);
    ws.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    // the numerator weights p * v_scale as a bf16 pair hi + lo (16 significant
    // bits): the output is sum_j p_j (v_scale_j code_j) / sum_j p_j to about
    // 2^-17 relative, a convex combination of the dequantised rows, so a
    // one-key row returns code * v_scale rounded once
    float wt[8];
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) wt[i] = p[i] * vs[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = pack_bf16x2(wt[2 * i], wt[2 * i + 1]);
        lo[i] = pack_bf16x2(wt[2 * i] - bf16_lo(hi[i]), wt[2 * i + 1] - bf16_hi(hi[i]));
    }
    const u32x4 pk_hi = {hi[0], hi[1], hi[2], hi[3]};
    const u32x4 pk_lo = {lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        const bf16x8 vcb = as_bf16x8_8(codes_to_bf16(vc[db][0], vc[db][1]));
        ws.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcb, as_bf16x8_8(pk_hi), ws.acc[db], 0, 0, 0);
        ws.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcb, as_bf16x8_8(pk_lo), ws.acc[db], 0, 0, 0);
    }
    // the stage's reads have returned (the MFMAs hold them): refill it with tile t + R
    if (t + R < w.n_tiles) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
        issue8(w, t + R, kS);
    }
}

template <int D, int R>
__device__ __forceinline__ void wave_tiles8(const Int8WaveItem<D>& w, WaveState<D>& ws) {
#pragma unroll
    for (int t = 0; t < R; ++t)
        if (t < w.n_tiles) issue8(w, t, t);
    for (int t = 0; t < w.n_tiles; t += R) {
        tile_step8<D, R, 0>(w, t, ws);
        if (t + 1 < w.n_tiles) tile_step8<D, R, 1>(w, t + 1, ws);
        if constexpr (R == 4) {
            if (t + 2 < w.n_tiles) tile_step8<D, R, 2>(w, t + 2, ws);
            if (t + 3 < w.n_tiles) tile_step8<D, R, 3>(w, t + 3, ws);
        }
    }
}

// What a work item needs before its first load: the sequence length, this
// lane's query fragments and the block ids of this wave's tiles.
template <int D>
struct Int8Inputs {
    int L_raw;
    int ids0, ids1;
    u32x4 qf[D / 32];
    u32x4 kn, vn;  // decode_append_int8: this lane's 8 values of the new K/V row
    PackInputs pk;  // sequences sharing the chunk
};

template <int D, int G>
__device__ __forceinline__ Int8Inputs<D> load_int8_inputs(const DecodeKernelArgs& p, int s, int g, int c) {
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = wave_id();
    Int8Inputs<D> in;
    in.L_raw = a.seq_lens[s];
    // Q^T fragment for MFMA cc: column lane % 16, dims (lane / 16) D/4 +
    // 8 cc + [0, 8), the dims of the lane's K codes; column h is head h of
    // sequence s (zero past G), or, for the first sequence of a run that may
    // pack, head h % G of sequence s + h / G
    in.pk = load_pack_inputs<G>(p, s, c);
    const int h = lane & 15, j = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool lead = in.pk.on && s % pack_width<G>() == 0;
    const int qs = lead ? s + h / G : s;
    const bool qv = lead ? qs < a.num_seqs : h < G;
    const uint16_t* qp =
        a.q + ((int64_t)min(qs, a.num_seqs - 1) * a.num_q_heads + g * G + h % G) * D + j * (D / 4);
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) in.qf[cc] = qv ? load16(qp + 8 * cc) : zero;
    const int32_t* table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    const int k0 = c * p.chunk;
    const int last = a.max_blocks_per_seq - 1;
    // (an empty table row, possible only when every sequence is empty, is not read)
    in.ids0 = last >= 0 ? table[min((k0 + kTile8 * (wave + kDecodeWaves * lane)) >> p.log2_block, last)] : -1;
    in.ids1 = last >= 0 && p.chunk > kTile8 * kDecodeWaves * kWave
                  ? table[min((k0 + kTile8 * (wave + kDecodeWaves * (lane + kWave))) >> p.log2_block, last)]
                  : 0;
    in.kn = in.vn = zero;
    if (a.k_new) {
        const int64_t row = ((int64_t)s * a.num_kv_heads + g) * D + (lane % (D / 8)) * 8;
        in.kn = load16(a.k_new + row);
        in.vn = load16(a.v_new + row);
    }
    return in;
}

template <int D, int G, int R, typename Prefetch>
__device__ __forceinline__ void decode_int8_item(const DecodeKernelArgs& p, DecodeShared<D, G>& sh,
                                                 const Int8Stages<D>& st, int s, int g, int c, int nchunks,
                                                 int64_t slot, const Int8Inputs<D>& in, Prefetch prefetch) {
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int k0 = c * p.chunk;
    const int L = clamp_len(in.L_raw, a.max_blocks_per_seq << p.log2_block);
    const int k1 = min(k0 + p.chunk, L);
    const int tiles = (k1 - k0 + kTile8 - 1) / kTile8;

    Int8WaveItem<D> w;
    w.a = &a;
    w.log2_block = p.log2_block;
    w.g = g;
    w.k0 = k0;
    w.kend = k1;
    w.wave = wave;
    w.lane = lane;
    w.n_tiles = tiles > wave ? (tiles - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
    w.ids0 = in.ids0;
    w.ids1 = in.ids1;
    w.L = L;
    w.append = a.k_new != nullptr;
    w.c = p.qk_scale_log2;
    w.tl = int8_lanes<D>(lane);
    w.st = st;

    WaveState<D> ws;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) ws.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws.m = -INFINITY;
    ws.l = 0.f;
    wait_all_vm();  // the item's inputs (block ids, q, the pack's lengths and ids) are in
    // sequences sharing the chunk: a member's item exits (its run's first
    // item decodes it, converting the chunk's codes once for the whole
    // pack); the first item keeps the columns of its pack
    const int lead = s - s % pack_width<G>();
    const uint32_t pack = pack_of<G>(p, in.pk, c);
    prefetch();  // the next item's inputs travel with this item's first tiles
    if (s != lead && ((pack >> (s - lead)) & 1)) return;
    const bool packed = s == lead && pack != 0;
    w.stream = __builtin_amdgcn_readfirstlane(packed ? 0 : 1) != 0;  // a shared pack's rows are read by other packs
    const int h = lane & 15;
    const bool keep = h < G || (packed && ((pack >> (h / G)) & 1));
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) w.qf[cc] = keep ? in.qf[cc] : u32x4{0u, 0u, 0u, 0u};
    w.kq = w.vq = u32x2{0u, 0u};
    w.ks_new = w.vs_new = 0.f;
    if (w.append) {  // every lane group of the wave holds the row: quantise it (the scheme of kv_append_int8)
        w.kq = quantize_piece<D / 8>(in.kn, &w.ks_new);
        w.vq = quantize_piece<D / 8>(in.vn, &w.vs_new);
    }
    wave_tiles8<D, R>(w, ws);
    // the packed finish's merge buffer ([4 waves][16][D] floats) takes the
    // code stages, its maxima and sums the V code stages
    static_assert(R * kDecodeWaves * kTile8 * D >= kDecodeWaves * 16 * D * (int)sizeof(float),
                  "the code stages hold the packed merge buffer");
    if (packed)
        finish_pack<D, G>(p, reinterpret_cast<float*>(st.k[0]), reinterpret_cast<float*>(st.v[0]), ws, lead, g, c,
                          pack);
    else
        finish_item<D, G>(p, sh, ws, s, g, nchunks, slot);
}

// R: LDS ring depth per wave.  R = 4: 132 KB of stages at D = 128, one
// workgroup per CU; R = 2: 66 KB, two workgroups per CU, so two waves share
// each SIMD and hide each other's stalls (the long-context decode runs about
// 1.4x faster than with R = 4).
template <int D, int G, int R>
__global__ __launch_bounds__(kDecodeThreads) void decode_int8_kernel(DecodeKernelArgs p, int32_t* prefix_out) {
    __shared__ DecodeShared<D, G> sh;
    __shared__ __attribute__((aligned(16))) int8_t sK[R][kDecodeWaves * kTile8 * D];
    __shared__ __attribute__((aligned(16))) int8_t sV[R][kDecodeWaves * kTile8 * D];
    __shared__ __attribute__((aligned(16))) float sS[R][kDecodeWaves * 2 * kTile8];
    Int8Stages<D> st;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        st.k[i] = sK[i];
        st.v[i] = sV[i];
        st.sc[i] = sS[i];
    }
    run_items<D, G>(
        p, sh, prefix_out, [&](int s, int g, int c) { return load_int8_inputs<D, G>(p, s, g, c); },
        [&](int s, int g, int c, int n, int64_t slot, const Int8Inputs<D>& in, auto prefetch) {
            decode_int8_item<D, G, R>(p, sh, st, s, g, c, n, slot, in, prefetch);
        });
}

}  // namespace

hipError_t launch_decode_int8(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    DecodeKernelArgs kp;
    kp.a = a;
    kp.chunk = pl.chunk;
    kp.log2_block = ilog2(a.block_size);
    kp.max_chunks = pl.max_chunks;
    kp.persistent = pl.persistent;
    kp.pack = pl.pack;
    kp.last_first = pl.last_first;
    kp.max_partials = pl.max_partials;
    char* ws = static_cast<char*>(a.workspace);
    kp.counters = pl.fused ? reinterpret_cast<int32_t*>(ws + pl.counter_offset) : nullptr;
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + pl.prefix_offset);
    kp.lse = reinterpret_cast<float*>(ws + pl.lse_offset);
    kp.part = reinterpret_cast<float*>(ws + pl.o_offset);
    kp.qk_scale_log2 = a.scale * kLog2e;
    const int G = a.num_q_heads / a.num_kv_heads;  // the ring depth follows from (D, G): plan_decode_int8
    if (a.head_dim == 128) {
        switch (G) {
            case 1: return launch_split<128, 1>(decode_int8_kernel<128, 1, 2>, kp, prefix, stream);
            case 2: return launch_split<128, 2>(decode_int8_kernel<128, 2, 2>, kp, prefix, stream);
            case 4: return launch_split<128, 4>(decode_int8_kernel<128, 4, 2>, kp, prefix, stream);
            default: return launch_split<128, 8>(decode_int8_kernel<128, 8, 4>, kp, prefix, stream);
        }
    }
    switch (G) {
        case 1: return launch_split<64, 1>(decode_int8_kernel<64, 1, 2>, kp, prefix, stream);
        case 2: return launch_split<64, 2>(decode_int8_kernel<64, 2, 2>, kp, prefix, stream);
        case 4: return launch_split<64, 4>(decode_int8_kernel<64, 4, 2>, kp, prefix, stream);
        default: return launch_split<64, 8>(decode_int8_kernel<64, 8, 2>, kp, prefix, stream);
    }
}

DecodePlan plan_decode_int8(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_seq_len, int64_t total_kv_tokens) {
    // workgroups that fit one CU (LDS, then 512 VGPRs per SIMD lane): ring 2
    // at D = 128 (two; ring 4 and one for G = 8, whose merge buffer is
    // larger), ring 2 at D = 64 (three)
    const int group = num_q_heads / num_kv_heads;
    const int ring = head_dim == 128 && group == 8 ? 4 : 2;
    const int wgs = head_dim == 128 ? (group == 8 ? 1 : 2) : 3;
    DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, total_kv_tokens,
                                kTile8, wgs);
    // a launch that packs sequences sharing a chunk takes chunks of at most
    // 2048 keys: a pack item then carries half of a 4096-key shared prefix,
    // and the persistent grid's workgroups stay evenly loaded (256 sequences
    // on a 4096-token prefix + 16 of 32K tokens: 568 us with the 4096-key
    // chunks the cost model picks, 435-447 us at 2048, 470 us at 1024)
    if (pl.pack)
        pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, total_kv_tokens, kTile8, wgs,
                         kInt8PackedChunk);
    pl.ring = ring;  // plan_decode decides packing (items beyond two rounds) and the in-kernel merge
    return pl;
}

}  // namespace pkv
